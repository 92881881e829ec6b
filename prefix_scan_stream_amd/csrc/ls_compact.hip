// ls_compact.hip -- fused, stable stream compaction in one pass (gfx950).
//
// The pages build compaction from three materialised steps: predicate flags, an
// exclusive scan of the flags giving every kept element its output index, and a
// scatter (geek-doc.cn parallel prefix scan page, section 一; pgsm.cn SIMT page,
// section 4.2, which also writes the count on the device).  Here the three steps
// are fused per tile and the flags and indices never leave the chip:
//   1. take a tile id in start order, load the tile with 128-bit loads;
//   2. evaluate the predicate in registers; count kept elements per run of 4,
//      scan the counts (DPP wave scan + LDS scan of the per-wave totals);
//   3. stage the kept elements in LDS at their rank inside the tile -- order is
//      kept, so the result is stable and unique;
//   4. the first wave looks back over the tile status words for the number of
//      elements kept by all earlier tiles (the tile's output offset);
//   5. copy the staged run from LDS to out[offset ...] with consecutive lanes on
//      consecutive addresses; the last tile writes the count.
// No atomics touch the data; the only atomics are the tile-id counter and the
// status words.  HBM traffic: n*4 bytes read, count*4 bytes written.
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

constexpr int CP_BLOCK = 256;
constexpr int CP_WAVES = CP_BLOCK / 64;
constexpr int CP_CHUNKS = 4;
constexpr int CP_TILE = CP_BLOCK * CP_CHUNKS * 4;  // 4096 elements, 16 KiB staged in LDS

// Count status words: flag in bits 63..62, count in bits 61..0.
constexpr uint64_t CNT_MASK = (uint64_t(1) << 62) - 1;
__device__ __forceinline__ uint64_t pack_count(uint32_t flag, uint64_t c)
{
    return (uint64_t(flag) << 62) | (c & CNT_MASK);
}

// Predicate through a 4-entry truth table indexed by the comparison outcome:
// 0 = greater, 1 = less, 2 = equal, 3 = unordered (a NaN is involved).
template <int DT>
__device__ __forceinline__ uint32_t pred_bit(uint32_t v, uint32_t t, uint32_t table)
{
    int state;
    if constexpr (DT == DT_FLOAT32) {
        const float a = __builtin_bit_cast(float, v), b = __builtin_bit_cast(float, t);
        state = (a < b) ? 1 : (a == b) ? 2 : (a > b) ? 0 : 3;
    } else if constexpr (DT == DT_INT32) {
        const int32_t a = int32_t(v), b = int32_t(t);
        state = (a < b) ? 1 : (a == b) ? 2 : 0;
    } else {
        state = (v < t) ? 1 : (v == t) ? 2 : 0;
    }
    return (table >> state) & 1u;
}

// Number of elements kept by all tiles before `tile` (>= 1).  Same walk as the
// scan's look-back: lanes above the highest lane holding a full prefix carry
// per-tile counts (each <= CP_TILE, so their sum fits 32 bits); the full prefix
// itself is a 62-bit count read from that lane.
__device__ int64_t lookback_count(const uint64_t* status, int64_t tile, WsHeader* hdr)
{
    const int lane = lane_id();
    int64_t excl = 0;
    int64_t last = tile - 1;
    int spins = 0;
    for (;;) {
        const int64_t idx = last - 63 + lane;
        const uint64_t w = (idx >= 0) ? status_load(status + idx) : pack_count(ST_PREFIX, 0);
        const uint32_t flag = uint32_t(w >> 62);
        const uint64_t empty = __ballot(flag == ST_EMPTY);
        const uint64_t full = __ballot(flag == ST_PREFIX);
        const int hi = full ? 63 - __builtin_clzll(full) : -1;
        const uint64_t needed = (hi >= 0) ? (~0ull << hi) : ~0ull;
        if (empty & needed) {
            if (++spins < LOOKBACK_SPIN_LIMIT) {
                __builtin_amdgcn_s_sleep(1);
                continue;
            }
            if (lane == 0)
                flag_error(hdr, WS_ERR_LOOKBACK_TIMEOUT);
            return excl;
        }
        const uint32_t part = (lane > hi) ? uint32_t(w & CNT_MASK) : 0u;
        const uint32_t sum = read_lane(wave_inclusive_scan<SumU32>(part), 63);
        excl += int64_t(sum);
        if (hi >= 0) {
            const uint32_t lo32 = __builtin_amdgcn_readlane(uint32_t(w), hi);
            const uint32_t hi32 = __builtin_amdgcn_readlane(uint32_t(w >> 32), hi);
            excl += int64_t(((uint64_t(hi32) << 32) | lo32) & CNT_MASK);
            return excl;
        }
        last -= 64;
    }
}

template <int DT, bool VEC>
__global__ __launch_bounds__(CP_BLOCK) void compact_kernel(const uint32_t* __restrict__ in,
                                                           uint32_t* __restrict__ out, int64_t n,
                                                           int64_t num_tiles, uint32_t thr,
                                                           uint32_t table, WsHeader* hdr,
                                                           uint64_t* status, int64_t* count)
{
    __shared__ uint32_t s_items[CP_TILE];
    __shared__ uint32_t s_tot[CP_CHUNKS][CP_WAVES];
    __shared__ uint32_t s_tile;
    __shared__ int64_t s_base;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (tid == 0)
        s_tile = take_tile_id(hdr);
    __syncthreads();
    const int64_t tile = s_tile;
    const int64_t tbase = tile * CP_TILE;

    Run4<uint32_t> r[CP_CHUNKS];
    uint32_t keep[CP_CHUNKS];  // bit k: element k of the run is kept
#pragma unroll
    for (int j = 0; j < CP_CHUNKS; ++j) {
        const int64_t idx = tbase + 4 * int64_t(j * CP_BLOCK + tid);
        r[j] = load_run<uint32_t, VEC>(in, idx, n, 0u);
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            m |= (idx + k < n ? pred_bit<DT>(r[j].v[k], thr, table) : 0u) << k;
        keep[j] = m;
    }

    uint32_t wex[CP_CHUNKS];
#pragma unroll
    for (int j = 0; j < CP_CHUNKS; ++j) {
        const uint32_t c = __builtin_popcount(keep[j]);
        const uint32_t inc = wave_inclusive_scan<SumU32>(c);
        wex[j] = inc - c;
        if (lane == 63)
            s_tot[j][wave] = inc;
    }
    __syncthreads();

    uint32_t pre[CP_CHUNKS];
    uint32_t agg = 0;
#pragma unroll
    for (int jj = 0; jj < CP_CHUNKS; ++jj) {
#pragma unroll
        for (int ww = 0; ww < CP_WAVES; ++ww) {
            if (ww == wave)
                pre[jj] = agg;
            agg += s_tot[jj][ww];
        }
    }

    // stage kept elements at their rank within the tile
#pragma unroll
    for (int j = 0; j < CP_CHUNKS; ++j) {
        uint32_t rank = pre[j] + wex[j];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (keep[j] & (1u << k))
                s_items[rank++] = r[j].v[k];
        }
    }

    if (wave == 0) {
        int64_t base = 0;
        if (tile == 0) {
            if (lane == 0)
                status_store(status, pack_count(ST_PREFIX, agg));
        } else {
            if (lane == 0)
                status_store(status + tile, pack_count(ST_AGGREGATE, agg));
            base = lookback_count(status, tile, hdr);
            if (lane == 0)
                status_store(status + tile, pack_count(ST_PREFIX, uint64_t(base) + agg));
        }
        if (lane == 0)
            s_base = base;
    }
    __syncthreads();
    const int64_t base = s_base;

    uint32_t* dst = out + base;
    for (uint32_t i = tid; i < agg; i += CP_BLOCK)
        dst[i] = s_items[i];
    if (tile == num_tiles - 1 && tid == 0)
        *count = base + int64_t(agg);
}

__global__ void store_i64_kernel(int64_t* p, int64_t v)
{
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *p = v;
}

// ------------------------------------------------------------------ host side

int64_t compact_tile_elems() { return CP_TILE; }

static int64_t cp_tiles(int64_t n) { return (n + CP_TILE - 1) / CP_TILE; }

size_t compact_workspace_bytes(int64_t n)
{
    int64_t tiles = cp_tiles(n);
    if (tiles < 1)
        tiles = 1;
    size_t bytes = sizeof(WsHeader) + size_t(tiles) * sizeof(uint64_t);
    return (bytes + 255) & ~size_t(255);
}

static uint32_t truth_table(int cmp)
{
    // bit 0: greater, bit 1: less, bit 2: equal, bit 3: unordered
    switch (cmp) {
    case 0: return 0x2u;  // <
    case 1: return 0x6u;  // <=
    case 2: return 0x1u;  // >
    case 3: return 0x5u;  // >=
    case 4: return 0x4u;  // ==
    case 5: return 0xBu;  // !=
    }
    return 0u;
}

hipError_t launch_compact(const void* in, void* out, int64_t* count, int64_t n, int dtype, int cmp,
                          uint32_t thr, void* ws, hipStream_t s)
{
    if (n == 0) {
        hipLaunchKernelGGL(store_i64_kernel, dim3(1), dim3(64), 0, s, count, int64_t(0));
        return hipGetLastError();
    }
    const int64_t tiles = cp_tiles(n);
    hipError_t e = clear_workspace(ws, tiles, s);
    if (e != hipSuccess)
        return e;
    auto* hdr = reinterpret_cast<WsHeader*>(ws);
    auto* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    const bool vec = (reinterpret_cast<uintptr_t>(in) & 15) == 0;
    const auto* pin = reinterpret_cast<const uint32_t*>(in);
    auto* pout = reinterpret_cast<uint32_t*>(out);
    const uint32_t table = truth_table(cmp);
    const dim3 grid(static_cast<uint32_t>(tiles)), block(CP_BLOCK);
#define LS_CP_LAUNCH(DT)                                                                          \
    do {                                                                                          \
        if (vec)                                                                                  \
            hipLaunchKernelGGL((compact_kernel<DT, true>), grid, block, 0, s, pin, pout, n, tiles, \
                               thr, table, hdr, status, count);                                   \
        else                                                                                      \
            hipLaunchKernelGGL((compact_kernel<DT, false>), grid, block, 0, s, pin, pout, n,      \
                               tiles, thr, table, hdr, status, count);                            \
    } while (0)
    switch (dtype) {
    case DT_INT32: LS_CP_LAUNCH(DT_INT32); break;
    case DT_UINT32: LS_CP_LAUNCH(DT_UINT32); break;
    default: LS_CP_LAUNCH(DT_FLOAT32); break;
    }
#undef LS_CP_LAUNCH
    return hipGetLastError();
}

}  // namespace ls
