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
#ifndef LS_CP_CHUNKS
#define LS_CP_CHUNKS 16
#endif
constexpr int CP_CHUNKS = LS_CP_CHUNKS;
constexpr int CP_TILE = CP_BLOCK * CP_CHUNKS * 4;  // 16384 elements (64 KiB staged in LDS) by default

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

// What decides the keep bit, and what is written for a kept element.
enum CompactSrc : int { SRC_CMP = 0, SRC_FLAGS = 1 };    // (x CMP thr) / flag byte != 0
enum CompactPay : int { PAY_VALUE = 0, PAY_INDEX = 1 };  // x itself / its index (uint32)

template <int DT, bool VEC, int SRC = SRC_CMP, int PAY = PAY_VALUE, bool FLAG4 = true>
__global__ __launch_bounds__(CP_BLOCK) void compact_kernel(const uint32_t* __restrict__ in,
                                                           uint32_t* __restrict__ out, int64_t n,
                                                           int64_t num_tiles, uint32_t thr,
                                                           uint32_t table, WsHeader* hdr,
                                                           uint64_t* status, int64_t* count,
                                                           const uint8_t* __restrict__ flags)
{
    constexpr int PARTS = CP_CHUNKS * CP_WAVES;  // (run, wave) kept counts per tile
    constexpr uint32_t RUN_STRIDE = CP_BLOCK * 16u;
    static_assert(PARTS <= 64, "the (run, wave) counts are scanned by one wave");
    __shared__ uint32_t s_items[CP_TILE];
    __shared__ uint32_t s_part[PARTS];
    __shared__ uint32_t s_tile;
    __shared__ uint32_t s_kept;
    __shared__ int64_t s_base;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    if (tid == 0)
        s_tile = take_tile_id(hdr);
    __syncthreads();
    const int64_t tile = s_tile;
    const int64_t tbase = tile * CP_TILE;
    const int64_t rem = n - tbase;
    const uint32_t valid = rem < CP_TILE ? uint32_t(rem) : uint32_t(CP_TILE);
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tbase, valid * 4u);
    const uint32_t voff = uint32_t(tid) * 16u;

    // 1. load; keep bits in registers (elements past n are never kept)
    constexpr bool LOAD_VALUES = (SRC == SRC_CMP) || (PAY == PAY_VALUE);
    Run4<uint32_t> r[CP_CHUNKS];
    uint32_t keep[CP_CHUNKS];  // bit k: element k of the run is kept
    if constexpr (LOAD_VALUES) {
#pragma unroll
        for (int j = 0; j < CP_CHUNKS; ++j)
            r[j] = VEC ? load_run_x4<uint32_t>(rin, voff, j * RUN_STRIDE)
                       : load_run_x1<uint32_t>(rin, voff, j * RUN_STRIDE);
    }
    uint32_t fl[CP_CHUNKS];  // flag bytes of a run (SRC_FLAGS)
    if constexpr (SRC == SRC_FLAGS) {
        const __amdgpu_buffer_rsrc_t rfl = make_rsrc(flags + tbase, valid);
#pragma unroll
        for (int j = 0; j < CP_CHUNKS; ++j) {
            const uint32_t b0 = 4u * uint32_t(j * CP_BLOCK + tid);
            // a dword that straddles the end of the range would read as 0 as a whole,
            // so the one run holding the last flag bytes of a ragged tile loads bytes
            if (FLAG4 && (b0 + 4u <= valid || b0 >= valid)) {
                fl[j] = __builtin_amdgcn_raw_buffer_load_b32(rfl, b0, 0, CACHE_NT);
            } else {
                uint32_t w = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(rfl, b0 + k, 0, CACHE_NT)) << (8 * k);
                fl[j] = w;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < CP_CHUNKS; ++j) {
        const uint32_t e0 = 4u * uint32_t(j * CP_BLOCK + tid);
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            uint32_t b;
            if constexpr (SRC == SRC_FLAGS)
                b = ((fl[j] >> (8 * k)) & 0xffu) != 0u;
            else
                b = pred_bit<DT>(r[j].v[k], thr, table);
            m |= (e0 + k < valid ? b : 0u) << k;
        }
        keep[j] = m;
    }

    // 2. counts per run, wave scan of the counts, (run, wave) counts to LDS
    uint32_t wex[CP_CHUNKS];
#pragma unroll
    for (int j = 0; j < CP_CHUNKS; ++j) {
        const uint32_t c = __builtin_popcount(keep[j]);
        const uint32_t inc = wave_inclusive_scan<SumU32>(c);
        wex[j] = inc - c;
        if (lane == 63)
            s_part[j * CP_WAVES + wave] = inc;
    }
    __syncthreads();

    // 3. wave 0: tile-local exclusive offsets of the (run, wave) parts; publish
    // the tile's count so later tiles can use it before this tile is done
    if (wave == 0) {
        const uint32_t v = lane < PARTS ? s_part[lane] : 0u;
        const uint32_t inc = wave_inclusive_scan<SumU32>(v);
        const uint32_t kept = read_lane(inc, 63);
        if (lane < PARTS)
            s_part[lane] = inc - v;
        if (lane == 0) {
            s_kept = kept;
            status_store(status_word(status, tile), CountCodec::pack(tile == 0 ? ST_PREFIX : ST_AGGREGATE, kept));
        }
    }
    __syncthreads();
    const uint32_t kept = s_kept;

    // 4. stage kept elements in LDS at their rank inside the tile (input order)
#pragma unroll
    for (int j = 0; j < CP_CHUNKS; ++j) {
        uint32_t rank = s_part[j * CP_WAVES + wave] + wex[j];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (keep[j] & (1u << k))
            {
                if constexpr (PAY == PAY_INDEX)
                    s_items[rank++] = uint32_t(tbase) + 4u * uint32_t(j * CP_BLOCK + tid) + k;
                else
                    s_items[rank++] = r[j].v[k];
            }
        }
    }

    // 5. wave 0: number of elements kept by all earlier tiles (the output offset)
    if (wave == 0) {
        int64_t base = 0;
        if (tile != 0) {
            base = int64_t(lookback<CountCodec>(status, tile, hdr));
            if (lane == 0)
                status_store(status_word(status, tile), CountCodec::pack(ST_PREFIX, uint64_t(base) + kept));
        }
        if (lane == 0)
            s_base = base;
    }
    __syncthreads();
    const int64_t base = s_base;

    // 6. contiguous copy LDS -> out[base ...]: 32-bit stores up to the first
    // 16-byte boundary of the output, then 128-bit stores, then a 32-bit tail
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + base, kept * 4u);
    if (VEC) {
        const uint32_t mis = uint32_t(reinterpret_cast<uintptr_t>(out + base) >> 2) & 3u;
        uint32_t head = (4u - mis) & 3u;
        head = head < kept ? head : kept;
        if (uint32_t(tid) < head)
            __builtin_amdgcn_raw_buffer_store_b32(s_items[tid], rout, uint32_t(tid) * 4u, 0, STORE_POLICY);
        const uint32_t groups = (kept - head) >> 2;
        for (uint32_t g = tid; g < groups; g += CP_BLOCK) {
            const uint32_t i = head + 4u * g;
            u32x4 w;
            w.x = s_items[i];
            w.y = s_items[i + 1];
            w.z = s_items[i + 2];
            w.w = s_items[i + 3];
            __builtin_amdgcn_raw_buffer_store_b128(w, rout, i * 4u, 0, STORE_POLICY);
        }
        const uint32_t i = head + 4u * groups + uint32_t(tid);
        if (i < kept)
            __builtin_amdgcn_raw_buffer_store_b32(s_items[i], rout, i * 4u, 0, STORE_POLICY);
    } else {
        for (uint32_t i = tid; i < kept; i += CP_BLOCK)
            __builtin_amdgcn_raw_buffer_store_b32(s_items[i], rout, i * 4u, 0, STORE_POLICY);
    }
    if (tile == num_tiles - 1 && tid == 0)
        *count = base + int64_t(kept);
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
    size_t bytes = sizeof(WsHeader) + size_t(tiles) * STATUS_SLOT_BYTES;
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

template <int DT, bool VEC, int SRC, int PAY, bool FLAG4>
static void launch_compact_kernel(dim3 grid, hipStream_t s, const uint32_t* in, uint32_t* out, int64_t n,
                                  int64_t tiles, uint32_t thr, uint32_t table, WsHeader* hdr,
                                  uint64_t* status, int64_t* count, const uint8_t* flags)
{
    hipLaunchKernelGGL((compact_kernel<DT, VEC, SRC, PAY, FLAG4>), grid, dim3(CP_BLOCK), 0, s, in, out, n,
                       tiles, thr, table, hdr, status, count, flags);
}

// src: SRC_CMP / SRC_FLAGS; pay: PAY_VALUE / PAY_INDEX
hipError_t launch_compact_general(const void* in, const uint8_t* flags, void* out, int64_t* count,
                                  int64_t n, int dtype, int cmp, uint32_t thr, int src, int pay,
                                  void* ws, hipStream_t s)
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
    const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    const bool flag4 = (reinterpret_cast<uintptr_t>(flags) & 3) == 0;
    const auto* pin = reinterpret_cast<const uint32_t*>(in);
    auto* pout = reinterpret_cast<uint32_t*>(out);
    const uint32_t table = truth_table(cmp);
    const dim3 grid(static_cast<uint32_t>(tiles));
#define LS_CP(DT, V, SRC, PAY, F4) \
    launch_compact_kernel<DT, V, SRC, PAY, F4>(grid, s, pin, pout, n, tiles, thr, table, hdr, status, count, flags)
    if (src == SRC_CMP) {
        if (pay == PAY_VALUE) {
            switch (dtype) {
            case DT_INT32: if (vec) LS_CP(DT_INT32, true, SRC_CMP, PAY_VALUE, true); else LS_CP(DT_INT32, false, SRC_CMP, PAY_VALUE, true); break;
            case DT_UINT32: if (vec) LS_CP(DT_UINT32, true, SRC_CMP, PAY_VALUE, true); else LS_CP(DT_UINT32, false, SRC_CMP, PAY_VALUE, true); break;
            default: if (vec) LS_CP(DT_FLOAT32, true, SRC_CMP, PAY_VALUE, true); else LS_CP(DT_FLOAT32, false, SRC_CMP, PAY_VALUE, true); break;
            }
        } else {
            switch (dtype) {
            case DT_INT32: if (vec) LS_CP(DT_INT32, true, SRC_CMP, PAY_INDEX, true); else LS_CP(DT_INT32, false, SRC_CMP, PAY_INDEX, true); break;
            case DT_UINT32: if (vec) LS_CP(DT_UINT32, true, SRC_CMP, PAY_INDEX, true); else LS_CP(DT_UINT32, false, SRC_CMP, PAY_INDEX, true); break;
            default: if (vec) LS_CP(DT_FLOAT32, true, SRC_CMP, PAY_INDEX, true); else LS_CP(DT_FLOAT32, false, SRC_CMP, PAY_INDEX, true); break;
            }
        }
    } else {
        if (pay == PAY_VALUE) {
            if (vec) { if (flag4) LS_CP(DT_UINT32, true, SRC_FLAGS, PAY_VALUE, true); else LS_CP(DT_UINT32, true, SRC_FLAGS, PAY_VALUE, false); }
            else { if (flag4) LS_CP(DT_UINT32, false, SRC_FLAGS, PAY_VALUE, true); else LS_CP(DT_UINT32, false, SRC_FLAGS, PAY_VALUE, false); }
        } else {
            if (vec) { if (flag4) LS_CP(DT_UINT32, true, SRC_FLAGS, PAY_INDEX, true); else LS_CP(DT_UINT32, true, SRC_FLAGS, PAY_INDEX, false); }
            else { if (flag4) LS_CP(DT_UINT32, false, SRC_FLAGS, PAY_INDEX, true); else LS_CP(DT_UINT32, false, SRC_FLAGS, PAY_INDEX, false); }
        }
    }
#undef LS_CP
    return hipGetLastError();
}

hipError_t launch_compact(const void* in, void* out, int64_t* count, int64_t n, int dtype, int cmp,
                          uint32_t thr, void* ws, hipStream_t s)
{
    return launch_compact_general(in, nullptr, out, count, n, dtype, cmp, thr, SRC_CMP, PAY_VALUE, ws, s);
}

}  // namespace ls
