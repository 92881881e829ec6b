// ls_compact.hip -- fused, stable stream compaction in one pass (gfx950).
//
// The pages build compaction from three materialised steps: predicate flags, an
// exclusive scan of the flags giving every kept element its output index, and a
// scatter (geek-doc.cn parallel prefix scan page, section 一; pgsm.cn SIMT page,
// section 4.2, which also writes the count on the device).  Here the three steps
// are fused per tile and the flags and indices never leave the chip:
//   1. a tile (16384 elements) is loaded with 128-bit loads into registers;
//   2. the predicate is evaluated in registers; kept elements are counted per run
//      of 4 and the counts scanned (DPP wave scan, then one wave over the
//      (run, wave) counts); the tile's total is published at once;
//   3. the kept elements are staged in LDS at their rank inside the tile -- order
//      is kept, so the result is stable and unique;
//   4. a control wave looks back over the tile status words for the number of
//      elements kept by all earlier tiles (the tile's output offset), 8 words per
//      poll, or 32 for a tile that moves little data;
//   5. the staged run is copied from LDS to out[offset ...] with consecutive
//      lanes on consecutive addresses; the last tile writes the count.
// Blocks are persistent and pipelined: the next tile's loads and count run while
// the current tile's look-back does.  No atomics touch the data; the only
// atomics are the status words and the count of started blocks.  HBM traffic:
// n*4 bytes read, count*4 bytes written.
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

#ifndef LS_CP_BLOCK
#define LS_CP_BLOCK 512
#endif
constexpr int CP_BLOCK = LS_CP_BLOCK;               // data threads per block
constexpr int CP_WAVES = CP_BLOCK / 64;             // data waves
constexpr int CP_THREADS = CP_BLOCK + 64;           // data waves + one control wave
#ifndef LS_CP_CHUNKS
#define LS_CP_CHUNKS 8
#endif
constexpr int CP_CHUNKS = LS_CP_CHUNKS;             // 16-byte runs per data thread
constexpr int CP_TILE = CP_BLOCK * CP_CHUNKS * 4;   // 16384 elements (64 KiB staged in LDS) by default
constexpr int CP_LB_WIDE = 8;                       // status words per look-back poll
// A tile that moves little data -- its loads plus 4 bytes per kept element under
// CP_SPARSE_BYTES -- polls 32 words at a time: it reaches a published prefix in
// fewer round trips, while for the others wide polls compete with the data stream.
// Measured on MI355X, 2^27 elements: compact_if 109 / 118 / 137 / 178 us at 1 / 20 /
// 50 / 99 % kept, against 113 / 120 / 137 / 179 us with 8 words for every tile (32
// words for every tile: 146 / 208 us at 50 / 99 %); index selection by flags 103 /
// 128 / 138 us at 50 / 80 / 98 %, against 117 / 130 / 138 us with 8 words.  A tile of
// flags loads 16 KiB, so its cut falls at 87.5 % kept; a tile of values loads 64 KiB:
// 12.5 %.
constexpr int CP_LB_WIDE_SPARSE = 32;
constexpr uint32_t CP_SPARSE_BYTES = 72 * 1024;

// Predicate through a 4-entry truth table indexed by the comparison outcome:
// 0 = greater, 1 = less, 2 = equal, 3 = unordered (a NaN is involved).
template <int DT>
__device__ __forceinline__ uint32_t pred_bit(uint32_t v, uint32_t t, uint32_t table)
{
    int state;
    if constexpr (DT == DT_FLOAT32) {
        // IEEE order through integer keys: -0 is folded into +0, a NaN on either
        // side is unordered, and the sign-magnitude bits map to an unsigned key
        // that orders like the values (negative: all bits flipped; otherwise:
        // the sign bit set).  Same outcomes as float compares, fewer registers.
        auto key = [](uint32_t u) -> uint32_t {
            u = (u << 1) == 0u ? 0u : u;
            return u ^ (uint32_t(int32_t(u) >> 31) | 0x80000000u);
        };
        const bool nan = (v & 0x7fffffffu) > 0x7f800000u || (t & 0x7fffffffu) > 0x7f800000u;
        const uint32_t a = key(v), b = key(t);
        state = nan ? 3 : (a < b) ? 1 : (a == b) ? 2 : 0;
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

// The staging buffer is dynamic LDS so that the compiler's occupancy model does
// not cap the register budget by it: with the buffer static the compiler aimed at
// one block per CU and used up to 168 VGPRs; dynamic, it fits two (at most 128).
#ifdef LS_CP_WPE
#define LS_CP_WAVES_ATTR __attribute__((amdgpu_waves_per_eu(LS_CP_WPE)))
#else
#define LS_CP_WAVES_ATTR
#endif

// Persistent blocks of CP_WAVES data waves and one control wave; a tile is
// 16384 elements, staged whole in 64 KiB of LDS, two blocks per CU.  Block b of
// G handles tiles b, b + G, b + 2G, ... (tile ids by block index: no counter);
// its tiles are numbered k = 0, 1, ... in that order.  At the top of step k, tile
// k is counted (its tile-local offsets and total are in LDS).
//   data waves: stage tile k's kept elements at their ranks, run by run, each
//     run's registers then taking tile k+1's run, so its loads start with the
//     staging; count tile k+1 -- the last data wave to finish scans the
//     (run, wave) counts and publishes the tile's total at once.
//   control wave, meanwhile: tile k's output offset by look-back; publish the
//     full prefix.
//   [barrier]  data waves: copy tile k out.  [barrier]
// The look-back and the copy run while tile k+1 loads.  A look-back that waits
// longer than the fallback time counts the missing tiles itself, so a block that
// is not yet resident costs time, never a wrong result; the grid is capped at the
// blocks that are resident at once all the same (resident_blocks below).
// 16384-element tiles, two blocks per CU, measured 113 / 137 / 178 us on MI355X
// with 8-word look-back polls for every tile
// (2^27 int32, 1 / 50 / 99 % kept) against 109 / 145 / 191 us for 32768-element
// tiles, one block per CU.
template <int DT, bool VEC, int SRC = SRC_CMP, int PAY = PAY_VALUE, bool FLAG4 = true>
LS_CP_WAVES_ATTR __global__ __launch_bounds__(CP_THREADS) void compact_kernel(const uint32_t* __restrict__ in,
                                                             uint32_t* __restrict__ out, int64_t n,
                                                             int64_t num_tiles, uint32_t thr,
                                                             uint32_t table, WsHeader* hdr,
                                                             uint64_t* status, int64_t* count,
                                                             const uint8_t* __restrict__ flags)
{
    constexpr int PARTS = CP_CHUNKS * CP_WAVES;  // (run, wave) kept counts per tile, in element order
    constexpr int PPL = (PARTS + 63) / 64;       // parts per lane in their scan
    constexpr uint32_t RUN_STRIDE = CP_BLOCK * 16u;
    constexpr bool LOAD_VALUES = (SRC == SRC_CMP) || (PAY == PAY_VALUE);
    constexpr uint32_t TILE_LOAD_BYTES = (LOAD_VALUES ? 4u * CP_TILE : 0u) + (SRC == SRC_FLAGS ? uint32_t(CP_TILE) : 0u);
    static_assert(PARTS <= 64 * PPL, "the (run, wave) counts are scanned by one wave, PPL per lane");
    static_assert((CP_WAVES & (CP_WAVES - 1)) == 0, "arrival counting takes CP_WAVES a power of two");
    static_assert(CP_CHUNKS <= 16, "keep bits of all runs fit in 64 bits");
    extern __shared__ uint32_t s_items[];  // CP_TILE words, sized at launch
    __shared__ uint32_t s_part[2][PARTS];  // tile k's offsets while tile k+1 is counted
    __shared__ uint32_t s_kept[2];
    __shared__ uint32_t s_arrive;          // data waves done counting (all tiles so far)
    __shared__ int64_t s_next[2];          // id of tile k+1, by step parity
    __shared__ int64_t s_base;
    __shared__ uint32_t s_ep;              // the call's epoch (the same in every ticket of the call)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const bool ctrl = wave == CP_WAVES;
    const uint32_t voff = uint32_t(tid) * 16u;

    auto tile_valid = [&](int64_t t) -> uint32_t {
        const int64_t rem = n - t * CP_TILE;
        return rem < CP_TILE ? uint32_t(rem) : uint32_t(CP_TILE);
    };

    Run4<uint32_t> r[CP_CHUNKS];
    uint32_t fl[CP_CHUNKS];  // flag bytes of a run (SRC_FLAGS)
    // packed to spare registers: keep bits 4j..4j+3 = elements of run j kept;
    // byte j of wex[j / 4] = kept elements of run j in lower lanes of the wave
    // (at most 63 * 4 = 252)
    uint64_t keep = 0;
    uint32_t wex[(CP_CHUNKS + 3) / 4];

    // Loads of run j of tile t (values and / or flag bytes) into r[j] / fl[j].
    auto load_run = [&](int64_t t, int j) {
        const int64_t tb = t * CP_TILE;
        const uint32_t valid = tile_valid(t);
        if constexpr (LOAD_VALUES) {
            const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tb, valid * 4u);
            r[j] = VEC ? load_run_x4<uint32_t>(rin, voff, j * RUN_STRIDE)
                       : load_run_x1<uint32_t>(rin, voff, j * RUN_STRIDE);
        }
        if constexpr (SRC == SRC_FLAGS) {
            const __amdgpu_buffer_rsrc_t rfl = make_rsrc(flags + tb, valid);
            const uint32_t b0 = 4u * uint32_t(j * CP_BLOCK + tid);
            // a dword that straddles the end of the range would read as 0 as a
            // whole, so the one run holding the last flag bytes of a ragged tile
            // loads bytes
            if (FLAG4 && (b0 + 4u <= valid || b0 >= valid)) {
                fl[j] = __builtin_amdgcn_raw_buffer_load_b32(rfl, b0, 0, CACHE_NT);
            } else {
                uint32_t w = 0;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    w |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(rfl, b0 + q, 0, CACHE_NT)) << (8 * q);
                fl[j] = w;
            }
        }
    };

    // Keep bits, per-run counts and their wave scans.  The last data wave to arrive turns the (run, wave) counts into
    // tile-local offsets and publishes the tile's total; no block barrier is
    // needed, so counting overlaps the control wave's look-back.
    auto count_tile = [&](int64_t t, int buf) {
        const uint32_t valid = tile_valid(t);
        keep = 0;
#pragma unroll
        for (int j = 0; j < (CP_CHUNKS + 3) / 4; ++j)
            wex[j] = 0;
        // elements past n are never kept: only the block's ragged last tile masks,
        // with one clamp per run (per-element indices would be loop-invariant
        // registers the compiler keeps live across the whole loop)
        const bool ragged = valid < uint32_t(CP_TILE);
        const int32_t lim = int32_t(valid) - 4 * tid;  // run j holds lim - 4 j CP_BLOCK valid elements
#pragma unroll
        for (int j = 0; j < CP_CHUNKS; ++j) {
            uint32_t m = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t b;
                if constexpr (SRC == SRC_FLAGS)
                    b = ((fl[j] >> (8 * q)) & 0xffu) != 0u;
                else
                    b = pred_bit<DT>(r[j].v[q], thr, table);
                m |= b << q;
            }
            if (ragged) {
                const int32_t rj = lim - 4 * j * CP_BLOCK;
                m &= rj >= 4 ? 0xfu : rj <= 0 ? 0u : (1u << rj) - 1u;
            }
            keep |= uint64_t(m) << (4 * j);
        }
#pragma unroll
        for (int j = 0; j < CP_CHUNKS; ++j) {
            const uint32_t c = __builtin_popcount(uint32_t(keep >> (4 * j)) & 0xfu);
            const uint32_t inc = wave_inclusive_scan<SumU32>(c);
            wex[j / 4] |= (inc - c) << (8 * (j % 4));
            if (lane == 63)
                s_part[buf][j * CP_WAVES + wave] = inc;
        }
        uint32_t old = 0;
        if (lane == 63)  // the lane that wrote this wave's counts releases them
            old = __hip_atomic_fetch_add(&s_arrive, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
        old = __builtin_amdgcn_readlane(old, 63);
        if ((old & (CP_WAVES - 1)) == CP_WAVES - 1) {
            // lane l scans parts PPL l .. PPL l + PPL - 1; lanes past PARTS / PPL
            // hold none (their indices would run into the LDS words that follow)
            uint32_t v[PPL];
            uint32_t sum = 0;
#pragma unroll
            for (int q = 0; q < PPL; ++q) {
                const int i = PPL * lane + q;
                v[q] = i < PARTS ? s_part[buf][i] : 0u;
                sum += v[q];
            }
            const uint32_t inc = wave_inclusive_scan<SumU32>(sum);
            const uint32_t kept = read_lane(inc, 63);
            uint32_t ex = inc - sum;
#pragma unroll
            for (int q = 0; q < PPL; ++q) {
                const int i = PPL * lane + q;
                if (i < PARTS)
                    s_part[buf][i] = ex;
                ex += v[q];
            }
            if (lane == 0) {
                s_kept[buf] = kept;
                status_store(status_word(status, t),
                             CountCodec::pack(t == 0 ? ST_PREFIX : ST_AGGREGATE, kept, s_ep));
            }
        }
    };

    // Recount of full tile j by the control wave, for the fallback of a wait that
    // runs out of time (the tile's block may not have been dispatched yet).  A count
    // of kept elements does not depend on the order in which it is summed.
    auto recount = [&](int64_t j) -> uint64_t {
        const int64_t tb = j * CP_TILE;
        uint32_t c = 0;
        for (uint32_t q = uint32_t(lane); q < uint32_t(CP_TILE / 4); q += 64) {  // elements 4q .. 4q+3
            if constexpr (SRC == SRC_FLAGS) {
                const __amdgpu_buffer_rsrc_t rfl = make_rsrc(flags + tb, uint32_t(CP_TILE));
                uint32_t w = 0;
                if (FLAG4) {
                    w = __builtin_amdgcn_raw_buffer_load_b32(rfl, 4u * q, 0, CACHE_NT);
                } else {
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        w |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(rfl, 4u * q + b, 0, CACHE_NT)) << (8 * b);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    c += ((w >> (8 * b)) & 0xffu) != 0u;
            } else {
                const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tb, uint32_t(CP_TILE) * 4u);
                const Run4<uint32_t> v = VEC ? load_run_x4<uint32_t>(rin, 16u * q, 0) : load_run_x1<uint32_t>(rin, 16u * q, 0);
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    c += pred_bit<DT>(v.v[b], thr, table);
            }
        }
        return uint64_t(read_lane(wave_inclusive_scan<SumU32>(c), 63));
    };

    // Tiles go to the G blocks by index: block b handles tiles b, b + G, b + 2G, ...
    // Prologue: the first one, counted.
    if (tid == 0) {
        s_arrive = 0;
        s_ep = read_epoch(hdr);
    }
    __syncthreads();
    const uint32_t ep = s_ep;
    const int64_t nblk = gridDim.x;
    int64_t cur = blockIdx.x;
    if (cur >= num_tiles) {  // never with the launch's grid; uniform over the block
        if (tid == 0)
            mark_started(hdr);
        return;
    }
    if (!ctrl) {
#pragma unroll
        for (int j = 0; j < CP_CHUNKS; ++j)
            load_run(cur, j);
        count_tile(cur, 0);
        if (tid == 0) {
            s_next[0] = cur + nblk;
            mark_started(hdr);  // the epoch read completed before the barrier above (its LDS copy)
        }
    }
    __syncthreads();

    for (uint32_t k = 0;; ++k) {
        const int buf = int(k & 1);
        const int64_t tbase = cur * CP_TILE;
        const int64_t next = s_next[buf];
        const uint32_t kept = s_kept[buf];

        if (!ctrl) {
            // stage tile k at its ranks inside the tile (input order); each run's
            // registers then take tile k+1's run.  The two cases are separate loops
            // so that the compiler's wait counting sees every load consumed on its
            // path.
            auto stage_run = [&](int j) {
                const uint32_t kj = uint32_t(keep >> (4 * j)) & 0xfu;
                uint32_t rank = s_part[buf][j * CP_WAVES + wave] + ((wex[j / 4] >> (8 * (j % 4))) & 0xffu);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (kj & (1u << q)) {
                        if constexpr (PAY == PAY_INDEX)
                            s_items[rank++] = uint32_t(tbase) + 4u * uint32_t(j * CP_BLOCK + tid) + q;
                        else
                            s_items[rank++] = r[j].v[q];
                    }
                }
            };
            if (next < num_tiles) {
                const int64_t g = next + nblk;  // the block's tile after next
#pragma unroll
                for (int j = 0; j < CP_CHUNKS; ++j) {
                    stage_run(j);
                    load_run(next, j);
                }
                count_tile(next, buf ^ 1);
                if (tid == 0)
                    s_next[buf ^ 1] = g;
            } else {
#pragma unroll
                for (int j = 0; j < CP_CHUNKS; ++j)
                    stage_run(j);
            }
        } else {
            // the tile's place in the output: the kept elements of all earlier
            // tiles, by look-back (missing counts recounted here when out of time)
            int64_t base = 0;
            if (cur != 0) {
                base = TILE_LOAD_BYTES + 4u * kept < CP_SPARSE_BYTES
                           ? int64_t(lookback<CountCodec, CP_LB_WIDE_SPARSE>(status, cur, ep, hdr, recount))
                           : int64_t(lookback<CountCodec, CP_LB_WIDE>(status, cur, ep, hdr, recount));
                if (lane == 0)
                    status_store(status_word(status, cur), CountCodec::pack(ST_PREFIX, uint64_t(base) + kept, ep));
            }
            if (lane == 0) {
                s_base = base;
                if (cur == num_tiles - 1) {
                    *count = base + int64_t(kept);
                    end_call(hdr, ep, gridDim.x);
                }
            }
        }
        __syncthreads();  // tile k staged, its offset known, tile k+1 counted
        const int64_t base = s_base;

        if (!ctrl) {
            // contiguous copy LDS -> out[base ...]: 32-bit stores up to the first
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
        }
        __syncthreads();  // tile k copied out before tile k+1 is staged over it
        if (next >= num_tiles)
            break;
        cur = next;
    }
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

// Blocks of this kernel that fit on the device at once (the persistent grid),
// after allowing it its 128 KiB of dynamic LDS on the current device.  Any grid
// size is correct -- blocks take tiles from the counter until none are left -- so
// the figure only sets how many tiles are in flight.  Cached per device and per
// kernel (the kernels differ in registers); 0 on failure (the caller reports it).
constexpr int CP_MAX_DEVICES = 64;

template <int DT, bool VEC, int SRC, int PAY, bool FLAG4>
static uint32_t resident_blocks()
{
    auto* kernel = compact_kernel<DT, VEC, SRC, PAY, FLAG4>;
    static int cached[CP_MAX_DEVICES] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 0;
    const bool cacheable = dev >= 0 && dev < CP_MAX_DEVICES;
    int v = cacheable ? __atomic_load_n(&cached[dev], __ATOMIC_RELAXED) : 0;
    if (v == 0) {
        int cus = 0, per_cu = 0;
        hipFuncAttributes attr{};
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                                int(CP_TILE * sizeof(uint32_t))) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, CP_THREADS, CP_TILE * sizeof(uint32_t)) !=
                hipSuccess ||
            hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel)) != hipSuccess)
            return 0;
        // The occupancy query assumes a block's waves spread evenly over the four
        // SIMDs of a CU; placed unevenly, a block of CP_THREADS / 64 waves may take
        // ceil(waves / 4) slots of one SIMD.  Only as many blocks as fit that way
        // are counted, so that every block of the grid is resident at once (a
        // block that is not would leave the tiles after its own waiting on the
        // fallback).  Measured: flag compaction at 96 VGPRs (5 waves per SIMD)
        // had only 510 of 512 two-per-CU blocks resident.
        const int vgprs = attr.numRegs > 0 ? (attr.numRegs + 7) & ~7 : 512;
        const int per_simd = 512 / vgprs < 8 ? 512 / vgprs : 8;
        const int uneven = per_simd / ((CP_THREADS / 64 + 3) / 4);
        per_cu = per_cu < uneven ? per_cu : uneven;
        v = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
        if (cacheable)
            __atomic_store_n(&cached[dev], v, __ATOMIC_RELAXED);
    }
    return uint32_t(v);
}

template <int DT, bool VEC, int SRC, int PAY, bool FLAG4>
static hipError_t launch_compact_kernel(hipStream_t s, const uint32_t* in, uint32_t* out, int64_t n,
                                  int64_t tiles, uint32_t thr, uint32_t table, WsHeader* hdr,
                                  uint64_t* status, int64_t* count, const uint8_t* flags)
{
    auto* k = compact_kernel<DT, VEC, SRC, PAY, FLAG4>;
    const uint32_t cap = resident_blocks<DT, VEC, SRC, PAY, FLAG4>();
    if (cap == 0)
        return hipErrorInvalidConfiguration;
    // at most as many blocks as are resident at once, so that none waits for a tile
    // whose block cannot start
    const uint32_t grid = tiles < int64_t(cap) ? uint32_t(tiles) : cap;
    hipLaunchKernelGGL(k, dim3(grid), dim3(CP_THREADS), CP_TILE * sizeof(uint32_t), s, in, out, n, tiles, thr,
                       table, hdr, status, count, flags);
    return hipGetLastError();
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
    hipError_t e = hipSuccess;
    auto* hdr = reinterpret_cast<WsHeader*>(ws);
    auto* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    const bool flag4 = (reinterpret_cast<uintptr_t>(flags) & 3) == 0;
    const auto* pin = reinterpret_cast<const uint32_t*>(in);
    auto* pout = reinterpret_cast<uint32_t*>(out);
    const uint32_t table = truth_table(cmp);
#define LS_CP(DT, V, SRC, PAY, F4) \
    e = launch_compact_kernel<DT, V, SRC, PAY, F4>(s, pin, pout, n, tiles, thr, table, hdr, status, count, flags)
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
    return e;
}

hipError_t launch_compact(const void* in, void* out, int64_t* count, int64_t n, int dtype, int cmp,
                          uint32_t thr, void* ws, hipStream_t s)
{
    return launch_compact_general(in, nullptr, out, count, n, dtype, cmp, thr, SRC_CMP, PAY_VALUE, ws, s);
}

}  // namespace ls
