// ls_scan.hip -- single-pass device-wide scan with decoupled look-back (gfx950).
//
// The parallel prefix scan page (geek-doc.cn, section 四) composes a large scan
// from per-block scans, a scan of the block totals, and a pass that adds each
// block's offset -- three launches, with the whole array read twice and written
// twice.  The same page mentions, and sets aside, letting blocks hand their
// totals to one another inside one launch through flags in global memory.  That
// is the design used here, because only it moves the minimum 2*n*4 bytes that
// bound an HBM-limited scan:
//   1. a block's tile is its block index (the fixed-order scheme instead takes
//      the next tile id from a counter, in the order blocks start); it loads the
//      tile (28672 elements; 16384 for the affine maps) with 128-bit loads;
//   2. it scans the tile in registers (serial runs of 4, DPP wave scan, one wave
//      over the (run, wave) totals) and publishes the tile total;
//   3. its first wave waits for the full prefix of the previous tile, which one
//      chasing wave publishes for every tile in order from the published totals
//      (the wave that scanned tile 0 stays on for this; see ls_device.hpp); a
//      tile that has waited a millisecond computes that prefix itself, since
//      the blocks it waits for may not have started;
//   4. it writes prefix (+) local scan with 128-bit stores.
// Each tile status is one 64-bit word (flag + value) so a single atomic access
// carries both; see ls_device.hpp.
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

#ifndef LS_SCAN_BLOCK
#define LS_SCAN_BLOCK 256
#endif
constexpr int SCAN_BLOCK = LS_SCAN_BLOCK;             // 4 waves by default
constexpr int SCAN_WAVES = SCAN_BLOCK / 64;
#ifndef LS_SCAN_CHUNKS
#define LS_SCAN_CHUNKS 16
#endif
constexpr int SCAN_CHUNKS = LS_SCAN_CHUNKS;           // 128-bit runs per thread
constexpr int SCAN_TILE = SCAN_BLOCK * SCAN_CHUNKS * 4;  // 16384 elements (three-phase schemes)

static_assert(SCAN_WAVES * SCAN_CHUNKS <= 64, "the (run, wave) totals are scanned by one wave");

// The single pass uses 8-wave blocks.  A tile holds its data in registers until
// its prefix is known, so the tile size sets how long the pipeline of resident
// tiles takes to fill and drain (two blocks per CU: 512 tiles), against the
// number of tiles the chasing wave must cover.  With tiles by block index, 14 runs
// per thread (28672-element tiles) measured best: 2^28 in 322-323 us, against
// 325-326 for 13 runs, 323-324 for 15, 334-336 for 16 and 346 / 377 for 10 / 8
// (float32 sum of 2^26: 83.5-84, 84-84.5, 85, 87 and 90 / 94.5 us).  While tiles
// took their ids from a counter atomic, 13 runs had been best (338-340 us against
// 341-343 for 12 and 14).  The deterministic scheme keeps 16 runs: its fixed groups of 64
// tiles are slower with smaller tiles (float32 2^26: 98 against 100-102 us).
// 16-wave blocks with 65536-element tiles (one block per CU) were slower
// (373-381 us).
#ifndef LS_SP_BLOCK
#define LS_SP_BLOCK 512
#endif
constexpr int SP_BLOCK = LS_SP_BLOCK;
constexpr int SP_WAVES = SP_BLOCK / 64;
#ifndef LS_SP_CHUNKS
#define LS_SP_CHUNKS 14
#endif
constexpr int SP_CHUNKS = LS_SP_CHUNKS;
constexpr int SP_TILE = SP_BLOCK * SP_CHUNKS * 4;          // 28672 elements
constexpr int SP_FIXED_TILE = SP_BLOCK * SCAN_CHUNKS * 4;  // 32768 elements (deterministic)

// Runs per thread of the single pass, by operator.  The affine maps' combine costs
// more registers: at 13 runs the kernel needs 151 VGPRs (one block per CU), at 8
// runs 106 (two).  MI355X, inclusive affine scan of 2^26: 99-100 us with 8 runs
// against 110-113 us for 32768-element tiles walking back over 8 status words per
// poll (one block per CU), and 115 us for 13 runs with chased prefixes.
constexpr int SP_AFF_CHUNKS = SP_CHUNKS < 8 ? SP_CHUNKS : 8;
template <class Op> constexpr int sp_chunks = SP_CHUNKS;
template <> constexpr int sp_chunks<AffU32> = SP_AFF_CHUNKS;
// The workspace holds a status slot for every tile of the smallest single-pass
// tile (run_scan checks this at compile time).
constexpr int SP_MIN_TILE = SP_BLOCK * SP_AFF_CHUNKS * 4;  // 16384 elements

// Tile-local part of the scan, shared by every tile a block processes: serial
// scan of each run, wave scan of the run totals (exclusive result in wex), and
// the (run, wave) totals left in LDS by lane 63, in element order.
template <class Op, int CHUNKS = SCAN_CHUNKS, int WAVES = SCAN_WAVES>
__device__ __forceinline__ void scan_tile_local(Run4<typename Op::T> (&r)[CHUNKS],
                                                typename Op::T (&wex)[CHUNKS],
                                                typename Op::T* s_part, int lane, int wave)
{
    using T = typename Op::T;
#pragma unroll
    for (int j = 0; j < CHUNKS; ++j) {
        r[j].v[1] = Op::apply(r[j].v[0], r[j].v[1]);
        r[j].v[2] = Op::apply(r[j].v[1], r[j].v[2]);
        r[j].v[3] = Op::apply(r[j].v[2], r[j].v[3]);
        const T inc = wave_inclusive_scan<Op>(r[j].v[3]);
        wex[j] = wave_shift_up<Op>(inc);
        if (lane == 63)
            s_part[j * WAVES + wave] = inc;
    }
}

#ifndef LS_SCAN_LDS_RESERVE
#define LS_SCAN_LDS_RESERVE 0
#endif

// The total of full tile j, computed by one wave with the same operations in the
// same order as tile j's own block (serial runs of 4, a wave scan over each
// (run, wave) row of run totals, the parts combined PPL per lane and scanned
// across one wave), so that float totals match bit for bit.  The fallback of a
// block-index tile whose wait ran out of time (replay_prefix).
template <class Op, bool VEC, int CHUNKS>
__device__ typename Op::T tile_total_by_wave(const typename Op::T* in, int64_t j)
{
    using T = typename Op::T;
    constexpr int PARTS = CHUNKS * SP_WAVES;
    constexpr int PPL = (PARTS + 63) / 64;
    constexpr int TILE = SP_BLOCK * CHUNKS * 4;
    constexpr uint32_t RUN_STRIDE = SP_BLOCK * 16u;
    const int lane = lane_id();
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + j * TILE, uint32_t(TILE) * 4u);
    T pv[PPL];
#pragma unroll
    for (int q = 0; q < PPL; ++q)
        pv[q] = Op::identity();
    for (int c = 0; c < CHUNKS; ++c) {
        for (int w = 0; w < SP_WAVES; ++w) {
            const uint32_t voff = uint32_t(w * 64 + lane) * 16u;
            const Run4<T> r = VEC ? load_run_x4<T>(rin, voff, c * RUN_STRIDE) : load_run_x1<T>(rin, voff, c * RUN_STRIDE);
            const T v1 = Op::apply(r.v[0], r.v[1]);
            const T v2 = Op::apply(v1, r.v[2]);
            const T v3 = Op::apply(v2, r.v[3]);
            const T part = read_lane(wave_inclusive_scan<Op>(v3), 63);
            const int p = c * SP_WAVES + w;
#pragma unroll
            for (int q = 0; q < PPL; ++q)
                pv[q] = (PPL * lane + q == p) ? part : pv[q];  // a select: no run-time register index
        }
    }
    T v = Op::identity();
#pragma unroll
    for (int q = 0; q < PPL; ++q)
        v = Op::apply(v, pv[q]);
    return read_lane(wave_inclusive_scan<Op>(v), 63);
}

// One tile per block.  The chased scans (BY_INDEX: every scan but the fixed-order
// one) take tile = block index.  FIXED takes tile ids in the order blocks start
// (tickets), and its look-back combines a fixed set of words in a fixed order
// (lookback_grouped), so float results are the same bits on every run.
template <class Op, bool INCLUSIVE, bool VEC, int CHUNKS, bool FIXED = false>
__global__ __launch_bounds__(SP_BLOCK) void scan_single_pass_kernel(
    const typename Op::T* in, typename Op::T* out, int64_t n, int64_t num_tiles, WsHeader* hdr,
    uint64_t* status, typename Op::T* total)
{
    using T = typename Op::T;
    using Codec = ScanCodec<Op>;
    constexpr bool BY_INDEX = !FIXED;
    constexpr int PARTS = CHUNKS * SP_WAVES;  // (run, wave) partial totals per tile
    constexpr int PPL = (PARTS + 63) / 64;    // partial totals per lane in their scan
    constexpr int TILE = SP_BLOCK * CHUNKS * 4;
    constexpr uint32_t RUN_STRIDE = SP_BLOCK * 16u;
    static_assert(PARTS % PPL == 0 && PARTS / PPL <= 64, "the (run, wave) totals are scanned by one wave");
    __shared__ T s_part[PARTS + LS_SCAN_LDS_RESERVE];
    __shared__ uint64_t s_ticket;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const T id = Op::identity();

    int64_t tile;
    uint32_t ep = 0;
    if constexpr (BY_INDEX) {
        // Thread 0 reads the epoch and the block waits for it before loading: the
        // loads of all eight waves then start together (measured, int32 scan of
        // 2^28: 326-327 us, against 334 us with each wave loading at once).
        tile = blockIdx.x;
        if (tid == 0)
            s_ticket = read_epoch(hdr);
        __syncthreads();
        ep = uint32_t(s_ticket);
    } else {
        if (tid == 0) {
            const uint64_t tk = take_ticket(hdr);
            s_ticket = tk;
            if (ticket_tile(tk) == num_tiles - 1)
                start_next_epoch(hdr, ticket_epoch(tk));  // the call's last ticket is out
            else if (ticket_tile(tk) >= num_tiles)
                flag_error(hdr, WS_ERR_BAD_TICKET);
        }
        __syncthreads();
        const uint64_t ticket = s_ticket;
        tile = ticket_tile(ticket);
        ep = ticket_epoch(ticket);
        if (tile >= num_tiles)
            return;  // uniform over the block: a workspace that was not initialised
    }
    const int64_t tbase = tile * TILE;
    const int64_t rem = n - tbase;
    const uint32_t valid = rem < TILE ? uint32_t(rem) : uint32_t(TILE);
    const bool full = valid == TILE;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tbase, valid * 4u);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + tbase, valid * 4u);
    const uint32_t voff = uint32_t(tid) * 16u;  // run j of thread t: elements 4*(j*BLOCK + t) + 0..3

    // 1. load.  Elements past n (last tile only) read as 0 (the buffer range is
    // checked per 32-bit word); they sit after every valid element in scan order,
    // so no output below n depends on them.
    Run4<T> r[CHUNKS];
#pragma unroll
    for (int j = 0; j < CHUNKS; ++j)
        r[j] = VEC ? load_run_x4<T>(rin, voff, j * RUN_STRIDE) : load_run_x1<T>(rin, voff, j * RUN_STRIDE);

    // 2. local scan: runs, wave scan of run totals, (run, wave) totals to LDS
    T wex[CHUNKS];
    scan_tile_local<Op, CHUNKS, SP_WAVES>(r, wex, s_part, lane, wave);
    __syncthreads();

    // 3. wave 0: scan the partial totals (one per lane), publish the tile total,
    // obtain the tile prefix, and leave prefix (+) partial-exclusive in LDS.
    T agg0 = id;  // tile 0's total: where the chasing wave starts
    if (wave == 0) {
        // lane l holds partial totals PPL l .. PPL l + PPL - 1, combined in order
        T pv[PPL];
        T v = id;
#pragma unroll
        for (int q = 0; q < PPL; ++q) {
            pv[q] = PPL * lane + q < PARTS ? s_part[PPL * lane + q] : id;
            v = Op::apply(v, pv[q]);
        }
        const T inc = wave_inclusive_scan<Op>(v);
        const T exc = wave_shift_up<Op>(inc);
        const T agg = read_lane(inc, 63);
        T p = id;
        if constexpr (FIXED) {
            // only the last tile of a group publishes a full prefix, the others
            // their totals (read by the later tiles of their group)
            const bool last_of_group = tile % LB_GROUP == LB_GROUP - 1;
            if (lane == 0 && !last_of_group)
                status_store(status_word(status, tile), Codec::pack(ST_AGGREGATE, agg, ep));
            if (tile != 0)
                p = lookback_grouped<Codec>(status, tile, ep, hdr);
            if (lane == 0 && last_of_group)
                status_store(status_word(status, tile), Codec::pack(ST_PREFIX, Op::apply(p, agg), ep));
        } else if constexpr (BY_INDEX) {
            if (lane == 0) {
                status_store(total_word(status, tile), Codec::pack(ST_AGGREGATE, agg, ep));
                if (tile == 0)
                    status_store(status, Codec::pack(ST_PREFIX, agg, ep));
            }
            bool replayed = false;
            if (tile == 0) {
                agg0 = agg;
            } else if (!wait_prefix<Codec>(status, tile, ep, p, FALLBACK_TICKS)) {
                // out of time (the tile before may not even have been dispatched):
                // compute the chasing wave's value here
                p = replay_prefix<Codec>(status, tile - 1, ep, [&](int64_t j) {
                    return tile_total_by_wave<Op, VEC, CHUNKS>(in, j);
                });
                replayed = true;
            }
            if (tile == num_tiles - 1) {  // every block has read the epoch: the next call may start a new one
                if (replayed)
                    await_totals<Codec>(status, tile, ep, hdr);
                if (lane == 0)
                    start_next_epoch(hdr, ep);
            }
        }
        T e = Op::apply(p, exc);
#pragma unroll
        for (int q = 0; q < PPL; ++q) {
            if (PPL * lane + q < PARTS)
                s_part[PPL * lane + q] = e;
            e = Op::apply(e, pv[q]);
        }
    }
    __syncthreads();

    // 4. finish and store; the thread holding element n-1 writes the total
    const int64_t last_local = (tile == num_tiles - 1) ? int64_t(valid) - 1 : -1;
#pragma unroll
    for (int j = 0; j < CHUNKS; ++j) {
        const T cp = Op::apply(s_part[j * SP_WAVES + wave], wex[j]);
        Run4<T> o;
        if constexpr (INCLUSIVE) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o.v[k] = Op::apply(cp, r[j].v[k]);
        } else {
            o.v[0] = cp;
#pragma unroll
            for (int k = 1; k < 4; ++k)
                o.v[k] = Op::apply(cp, r[j].v[k - 1]);
        }
        if (VEC && full)
            store_run_x4<T>(rout, voff, j * RUN_STRIDE, o);
        else
            store_run_x1<T>(rout, voff, j * RUN_STRIDE, o);
        if (total != nullptr) {
            // select, not index: a run-time index into r[] would move the whole
            // tile from registers to per-lane scratch memory
            const int64_t kk = last_local - 4 * int64_t(j * SP_BLOCK + tid);
            if (kk >= 0 && kk < 4) {
                T v = r[j].v[0];
#pragma unroll
                for (int k = 1; k < 4; ++k)
                    v = (kk == k) ? r[j].v[k] : v;
                *total = Op::apply(cp, v);
            }
        }
    }

    // 5. tile 0's first wave, its own tile written, publishes every later tile's
    // full prefix (it returns once the last tile's is out)
    if constexpr (BY_INDEX) {
        if (tile == 0 && wave == 0)
            chase_prefixes<Codec>(status, num_tiles, agg0, ep);
    }
}

// ---------------------------------------------------------------- three-phase
// The multi-block composition of the parallel prefix scan page (geek-doc.cn,
// section 四): scan each block, scan the block totals, add each block's offset.
// Kept beside the single pass so the two can be measured against each other.
//   reduce-then-scan   tile totals (read n) -> scan of totals -> seeded tile scan
//                      (read n, write n): 3n*4 bytes;
//   scan-then-propagate local tile scans + totals (read n, write n) -> scan of
//                      totals -> offsets added in place (read n, write n): 4n*4.
// No tile waits for another, so no status words and no tile counter; elements
// past n are replaced by the identity so every tile total is exact.

// Tile total: serial per thread over its runs, wave reduce, LDS across waves.
template <class Op, bool VEC>
__global__ __launch_bounds__(SCAN_BLOCK) void tile_reduce_kernel(const typename Op::T* in, int64_t n,
                                                                 typename Op::T* totals)
{
    using T = typename Op::T;
    __shared__ T s_w[SCAN_WAVES];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t tile = blockIdx.x;
    const int64_t rem = n - tile * SCAN_TILE;
    const uint32_t valid = rem < SCAN_TILE ? uint32_t(rem) : uint32_t(SCAN_TILE);
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tile * SCAN_TILE, valid * 4u);
    const uint32_t voff = uint32_t(tid) * 16u;
    if constexpr (Op::commutative) {
        // a thread folds its own runs (1024 elements apart), then the lanes and
        // the waves: out of element order, which only a commutative op allows
        T acc = Op::identity();
#pragma unroll
        for (int j = 0; j < SCAN_CHUNKS; ++j) {
            const Run4<T> r = VEC ? load_run_x4<T>(rin, voff, j * SCAN_BLOCK * 16u)
                                  : load_run_x1<T>(rin, voff, j * SCAN_BLOCK * 16u);
            const uint32_t e0 = 4u * uint32_t(j * SCAN_BLOCK + tid);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                acc = Op::apply(acc, e0 + k < valid ? r.v[k] : Op::identity());
        }
        const T inc = wave_inclusive_scan<Op>(acc);
        if (lane == 63)
            s_w[wave] = inc;
        __syncthreads();
        if (tid == 0) {
            T t = Op::identity();
#pragma unroll
            for (int w = 0; w < SCAN_WAVES; ++w)
                t = Op::apply(t, s_w[w]);
            totals[tile] = t;
        }
    } else {
        // element order: each run of 4, the runs of one chunk across the wave in
        // lane order, the (chunk, wave) parts chunk by chunk
        __shared__ T s_p[SCAN_CHUNKS * SCAN_WAVES];
#pragma unroll
        for (int j = 0; j < SCAN_CHUNKS; ++j) {
            const Run4<T> r = VEC ? load_run_x4<T>(rin, voff, j * SCAN_BLOCK * 16u)
                                  : load_run_x1<T>(rin, voff, j * SCAN_BLOCK * 16u);
            const uint32_t e0 = 4u * uint32_t(j * SCAN_BLOCK + tid);
            T run = Op::identity();
#pragma unroll
            for (int k = 0; k < 4; ++k)
                run = Op::apply(run, e0 + k < valid ? r.v[k] : Op::identity());
            const T inc = wave_inclusive_scan<Op>(run);
            if (lane == 63)
                s_p[j * SCAN_WAVES + wave] = inc;
        }
        __syncthreads();
        if (wave == 0) {
            constexpr int PARTS = SCAN_CHUNKS * SCAN_WAVES;
            static_assert(PARTS <= 64, "one wave combines the parts");
            const T inc = wave_inclusive_scan<Op>(lane < PARTS ? s_p[lane] : Op::identity());
            if (lane == 63)
                totals[tile] = inc;
        }
    }
}

// Tile scan with a given tile prefix: seeds[tile] when seeds != nullptr, else
// the identity; writes the tile total to totals[tile] when totals != nullptr.
template <class Op, bool INCLUSIVE, bool VEC>
__global__ __launch_bounds__(SCAN_BLOCK) void tile_scan_kernel(const typename Op::T* in,
                                                               typename Op::T* out, int64_t n,
                                                               const typename Op::T* seeds,
                                                               typename Op::T* totals)
{
    using T = typename Op::T;
    constexpr int PARTS = SCAN_CHUNKS * SCAN_WAVES;
    constexpr uint32_t RUN_STRIDE = SCAN_BLOCK * 16u;
    __shared__ T s_part[PARTS];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const T id = Op::identity();
    const int64_t tile = blockIdx.x;
    const int64_t tbase = tile * SCAN_TILE;
    const int64_t rem = n - tbase;
    const uint32_t valid = rem < SCAN_TILE ? uint32_t(rem) : uint32_t(SCAN_TILE);
    const bool full = valid == SCAN_TILE;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tbase, valid * 4u);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + tbase, valid * 4u);
    const uint32_t voff = uint32_t(tid) * 16u;

    Run4<T> r[SCAN_CHUNKS];
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j) {
        r[j] = VEC ? load_run_x4<T>(rin, voff, j * RUN_STRIDE) : load_run_x1<T>(rin, voff, j * RUN_STRIDE);
        if (!full) {
            const uint32_t e0 = 4u * uint32_t(j * SCAN_BLOCK + tid);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                r[j].v[k] = e0 + k < valid ? r[j].v[k] : id;
        }
    }
    T wex[SCAN_CHUNKS];
    scan_tile_local<Op>(r, wex, s_part, lane, wave);
    __syncthreads();
    if (wave == 0) {
        const T v = lane < PARTS ? s_part[lane] : id;
        const T inc = wave_inclusive_scan<Op>(v);
        const T exc = wave_shift_up<Op>(inc);
        const T p = seeds != nullptr ? seeds[tile] : id;
        if (totals != nullptr && lane == 0)
            totals[tile] = read_lane(inc, 63);
        if (lane < PARTS)
            s_part[lane] = Op::apply(p, exc);
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j) {
        const T cp = Op::apply(s_part[j * SCAN_WAVES + wave], wex[j]);
        Run4<T> o;
        if constexpr (INCLUSIVE) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o.v[k] = Op::apply(cp, r[j].v[k]);
        } else {
            o.v[0] = cp;
#pragma unroll
            for (int k = 1; k < 4; ++k)
                o.v[k] = Op::apply(cp, r[j].v[k - 1]);
        }
        if (VEC && full)
            store_run_x4<T>(rout, voff, j * RUN_STRIDE, o);
        else
            store_run_x1<T>(rout, voff, j * RUN_STRIDE, o);
    }
}

// out[i] = seeds[tile] (+) out[i] over each tile, in place.
template <class Op, bool VEC>
__global__ __launch_bounds__(SCAN_BLOCK) void add_offset_kernel(typename Op::T* out, int64_t n,
                                                                const typename Op::T* seeds)
{
    using T = typename Op::T;
    constexpr uint32_t RUN_STRIDE = SCAN_BLOCK * 16u;
    const int64_t tile = blockIdx.x;
    const int64_t tbase = tile * SCAN_TILE;
    const int64_t rem = n - tbase;
    const uint32_t valid = rem < SCAN_TILE ? uint32_t(rem) : uint32_t(SCAN_TILE);
    const bool full = valid == SCAN_TILE;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(out + tbase, valid * 4u);
    const uint32_t voff = uint32_t(threadIdx.x) * 16u;
    const T p = seeds[tile];
    Run4<T> r[SCAN_CHUNKS];
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j)
        r[j] = VEC ? load_run_x4<T>(rs, voff, j * RUN_STRIDE) : load_run_x1<T>(rs, voff, j * RUN_STRIDE);
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            r[j].v[k] = Op::apply(p, r[j].v[k]);
        if (VEC && full)
            store_run_x4<T>(rs, voff, j * RUN_STRIDE, r[j]);
        else
            store_run_x1<T>(rs, voff, j * RUN_STRIDE, r[j]);
    }
}

// total = seeds[last] (+) totals[last]
template <class Op>
__global__ void write_total_kernel(const typename Op::T* seeds, const typename Op::T* totals,
                                   int64_t last, typename Op::T* total)
{
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *total = Op::apply(seeds[last], totals[last]);
}

// Zero fill of a workspace (ls_workspace_init): 16-byte stores, a kernel rather
// than a memset so that the call can be captured in a graph.
__global__ __launch_bounds__(256) void ws_zero_kernel(u32x4* p, int64_t words)
{
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < words; i += int64_t(gridDim.x) * 256)
        p[i] = z;
}

__global__ void store_u32_kernel(uint32_t* p, uint32_t v)
{
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *p = v;
}

// ------------------------------------------------------------------ host side

int64_t scan_tile_elems() { return SCAN_TILE; }

static int64_t num_tiles_for(int64_t n) { return (n + SCAN_TILE - 1) / SCAN_TILE; }

static int64_t single_pass_tiles(int64_t n, bool fixed)
{
    const int64_t t = fixed ? SP_FIXED_TILE : SP_MIN_TILE;  // the smallest tile of each scheme
    return (n + t - 1) / t;
}

static size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// Single pass: header + one status word per tile.  Three-phase: tile totals and
// their scan (seeds), plus, when the totals span more than one tile, the
// workspace of the same scheme over the totals (the recursion of the page's
// multi-level scan).
size_t scan_workspace_bytes(int64_t n, int scheme)
{
    if (scheme == SCHEME_SINGLE_PASS || scheme == SCHEME_SINGLE_PASS_FIXED) {
        const int64_t sp = single_pass_tiles(n, scheme == SCHEME_SINGLE_PASS_FIXED);
        return round256(sizeof(WsHeader) + size_t(sp < 1 ? 1 : sp) * STATUS_SLOT_BYTES);
    }
    int64_t tiles = num_tiles_for(n);
    if (tiles < 1)
        tiles = 1;
    size_t bytes = 2 * round256(size_t(tiles) * 4);
    if (tiles > SCAN_TILE)
        bytes += scan_workspace_bytes(tiles, scheme);
    return bytes;
}

hipError_t init_workspace(void* ws, size_t bytes, hipStream_t s)
{
    const int64_t words = int64_t(bytes / 16);
    if (words == 0)
        return hipSuccess;
    int64_t blocks = (words + 255) / 256;
    blocks = blocks < 1024 ? blocks : 1024;
    hipLaunchKernelGGL(ws_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, reinterpret_cast<u32x4*>(ws), words);
    return hipGetLastError();
}

template <class Op>
static uint32_t identity_bits();
template <> uint32_t identity_bits<SumU32>() { return 0u; }
template <> uint32_t identity_bits<XorU32>() { return 0u; }
template <> uint32_t identity_bits<MaxU32>() { return 0u; }
template <> uint32_t identity_bits<MaxI32>() { return 0x80000000u; }
template <> uint32_t identity_bits<SumF32>() { return 0u; }
template <> uint32_t identity_bits<MaxF32>() { return 0xff800000u; }
template <> uint32_t identity_bits<MinU32>() { return 0xffffffffu; }
template <> uint32_t identity_bits<MinI32>() { return 0x7fffffffu; }
template <> uint32_t identity_bits<MinF32>() { return 0x7f800000u; }
template <> uint32_t identity_bits<AndU32>() { return 0xffffffffu; }
template <> uint32_t identity_bits<OrU32>() { return 0u; }
template <> uint32_t identity_bits<MulU32>() { return 1u; }
template <> uint32_t identity_bits<MulF32>() { return 0x3f800000u; }
template <> uint32_t identity_bits<AffU32>() { return 0x00010000u; }

template <class Op, int CHUNKS, bool FIXED = false>
static void launch_single_pass(const void* in, void* out, int64_t n, int64_t tiles, bool inclusive,
                               void* total, WsHeader* hdr, uint64_t* status, hipStream_t s)
{
    using T = typename Op::T;
    const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    const T* pin = reinterpret_cast<const T*>(in);
    T* pout = reinterpret_cast<T*>(out);
    T* ptot = reinterpret_cast<T*>(total);
    const dim3 grid(static_cast<uint32_t>(tiles)), block(SP_BLOCK);
    if (inclusive) {
        if (vec)
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, true, true, CHUNKS, FIXED>), grid, block, 0, s, pin,
                               pout, n, tiles, hdr, status, ptot);
        else
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, true, false, CHUNKS, FIXED>), grid, block, 0, s, pin,
                               pout, n, tiles, hdr, status, ptot);
    } else {
        if (vec)
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, false, true, CHUNKS, FIXED>), grid, block, 0, s, pin,
                               pout, n, tiles, hdr, status, ptot);
        else
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, false, false, CHUNKS, FIXED>), grid, block, 0, s, pin,
                               pout, n, tiles, hdr, status, ptot);
    }
}

// Tiles (status slots) of the single-pass uint32 sum over n elements.
int64_t scan_sum_u32_tiles(int64_t n) { return (n + SP_TILE - 1) / SP_TILE; }

// Exclusive uint32 sum by the single pass (n >= 1), for the radix sort.
hipError_t launch_scan_sum_u32_excl(const uint32_t* in, uint32_t* out, int64_t n, void* ws, hipStream_t s)
{
    auto* hdr = reinterpret_cast<WsHeader*>(ws);
    auto* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    launch_single_pass<SumU32, SP_CHUNKS, false>(in, out, n, scan_sum_u32_tiles(n), false, nullptr, hdr, status, s);
    return hipGetLastError();
}

template <class Op, bool FIXED = false>
static hipError_t run_scan(const void* in, void* out, int64_t n, bool inclusive, void* total,
                           void* ws, hipStream_t s)
{
    if (n == 0) {
        if (total)
            hipLaunchKernelGGL(store_u32_kernel, dim3(1), dim3(64), 0, s,
                               reinterpret_cast<uint32_t*>(total), identity_bits<Op>());
        return hipGetLastError();
    }
    constexpr int CHUNKS = FIXED ? SCAN_CHUNKS : sp_chunks<Op>;
    constexpr int64_t TILE = int64_t(SP_BLOCK) * CHUNKS * 4;
    static_assert(TILE >= (FIXED ? SP_FIXED_TILE : SP_MIN_TILE),
                  "a tile smaller than the workspace's would index status slots past its end");
    const int64_t tiles = (n + TILE - 1) / TILE;  // never more than the workspace holds
    auto* hdr = reinterpret_cast<WsHeader*>(ws);
    auto* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    launch_single_pass<Op, CHUNKS, FIXED>(in, out, n, tiles, inclusive, total, hdr, status, s);
    return hipGetLastError();
}

// Whether the fixed-order single pass is a kernel of its own for Op: where the
// association can change the bits (float sums and products), and for the affine
// maps, whose non-commutative combine lets the tests check the fixed order.  For
// the other operators every grouping gives the same bits, so the ordinary kernel
// serves.
template <class Op> constexpr bool fixed_order_kernel = false;
template <> constexpr bool fixed_order_kernel<SumF32> = true;
template <> constexpr bool fixed_order_kernel<MulF32> = true;
template <> constexpr bool fixed_order_kernel<AffU32> = true;

template <class Op>
static hipError_t run_three_phase(const typename Op::T* in, typename Op::T* out, int64_t n,
                                  bool inclusive, typename Op::T* total, char* ws, int scheme,
                                  hipStream_t s);

// Exclusive scan of the m tile totals into seeds: one block when they fit a
// tile, else the same scheme again over the totals.
template <class Op>
static hipError_t scan_totals(const typename Op::T* totals, typename Op::T* seeds, int64_t m,
                              char* sub_ws, int scheme, hipStream_t s)
{
    if (m <= SCAN_TILE) {
        hipLaunchKernelGGL((tile_scan_kernel<Op, false, true>), dim3(1), dim3(SCAN_BLOCK), 0, s,
                           totals, seeds, m, static_cast<const typename Op::T*>(nullptr),
                           static_cast<typename Op::T*>(nullptr));
        return hipGetLastError();
    }
    return run_three_phase<Op>(totals, seeds, m, false, nullptr, sub_ws, scheme, s);
}

template <class Op, bool INCLUSIVE>
static void launch_tile_scan(bool vec, const typename Op::T* in, typename Op::T* out, int64_t n,
                             int64_t tiles, const typename Op::T* seeds, typename Op::T* totals,
                             hipStream_t s)
{
    const dim3 grid(static_cast<uint32_t>(tiles)), block(SCAN_BLOCK);
    if (vec)
        hipLaunchKernelGGL((tile_scan_kernel<Op, INCLUSIVE, true>), grid, block, 0, s, in, out, n, seeds, totals);
    else
        hipLaunchKernelGGL((tile_scan_kernel<Op, INCLUSIVE, false>), grid, block, 0, s, in, out, n, seeds, totals);
}

template <class Op>
static hipError_t run_three_phase(const typename Op::T* in, typename Op::T* out, int64_t n,
                                  bool inclusive, typename Op::T* total, char* ws, int scheme,
                                  hipStream_t s)
{
    using T = typename Op::T;
    const int64_t tiles = num_tiles_for(n);
    T* totals = reinterpret_cast<T*>(ws);
    T* seeds = reinterpret_cast<T*>(ws + round256(size_t(tiles) * 4));
    char* sub = ws + 2 * round256(size_t(tiles) * 4);
    const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    const dim3 grid(static_cast<uint32_t>(tiles)), block(SCAN_BLOCK);
    hipError_t e;
    if (scheme == SCHEME_REDUCE_THEN_SCAN) {
        if (((reinterpret_cast<uintptr_t>(in)) & 15) == 0)
            hipLaunchKernelGGL((tile_reduce_kernel<Op, true>), grid, block, 0, s, in, n, totals);
        else
            hipLaunchKernelGGL((tile_reduce_kernel<Op, false>), grid, block, 0, s, in, n, totals);
        if ((e = scan_totals<Op>(totals, seeds, tiles, sub, scheme, s)) != hipSuccess)
            return e;
        if (inclusive)
            launch_tile_scan<Op, true>(vec, in, out, n, tiles, seeds, nullptr, s);
        else
            launch_tile_scan<Op, false>(vec, in, out, n, tiles, seeds, nullptr, s);
    } else {
        if (inclusive)
            launch_tile_scan<Op, true>(vec, in, out, n, tiles, nullptr, totals, s);
        else
            launch_tile_scan<Op, false>(vec, in, out, n, tiles, nullptr, totals, s);
        if ((e = scan_totals<Op>(totals, seeds, tiles, sub, scheme, s)) != hipSuccess)
            return e;
        if (((reinterpret_cast<uintptr_t>(out)) & 15) == 0)
            hipLaunchKernelGGL((add_offset_kernel<Op, true>), grid, block, 0, s, out, n, seeds);
        else
            hipLaunchKernelGGL((add_offset_kernel<Op, false>), grid, block, 0, s, out, n, seeds);
    }
    if (total != nullptr)
        hipLaunchKernelGGL((write_total_kernel<Op>), dim3(1), dim3(64), 0, s, seeds, totals, tiles - 1, total);
    return hipGetLastError();
}

template <class Op>
static hipError_t run_scan_scheme(const void* in, void* out, int64_t n, bool inclusive, void* total,
                                  void* ws, int scheme, hipStream_t s)
{
    using T = typename Op::T;
    if (scheme == SCHEME_SINGLE_PASS_FIXED && fixed_order_kernel<Op>)
        return run_scan<Op, fixed_order_kernel<Op>>(in, out, n, inclusive, total, ws, s);
    if (scheme == SCHEME_SINGLE_PASS || scheme == SCHEME_SINGLE_PASS_FIXED || n == 0)
        return run_scan<Op>(in, out, n, inclusive, total, ws, s);
    return run_three_phase<Op>(reinterpret_cast<const T*>(in), reinterpret_cast<T*>(out), n, inclusive,
                               reinterpret_cast<T*>(total), reinterpret_cast<char*>(ws), scheme, s);
}

hipError_t launch_scan(const void* in, void* out, int64_t n, int dtype, int op, bool inclusive,
                       void* total, void* ws, int scheme, hipStream_t s)
{
    switch (op) {
    case OP_SUM:
        if (dtype == DT_FLOAT32)
            return run_scan_scheme<SumF32>(in, out, n, inclusive, total, ws, scheme, s);
        return run_scan_scheme<SumU32>(in, out, n, inclusive, total, ws, scheme, s);
    case OP_XOR:
        return run_scan_scheme<XorU32>(in, out, n, inclusive, total, ws, scheme, s);
    case OP_MAX:
        if (dtype == DT_INT32)
            return run_scan_scheme<MaxI32>(in, out, n, inclusive, total, ws, scheme, s);
        if (dtype == DT_UINT32)
            return run_scan_scheme<MaxU32>(in, out, n, inclusive, total, ws, scheme, s);
        return run_scan_scheme<MaxF32>(in, out, n, inclusive, total, ws, scheme, s);
    case OP_MIN:
        if (dtype == DT_INT32)
            return run_scan_scheme<MinI32>(in, out, n, inclusive, total, ws, scheme, s);
        if (dtype == DT_UINT32)
            return run_scan_scheme<MinU32>(in, out, n, inclusive, total, ws, scheme, s);
        return run_scan_scheme<MinF32>(in, out, n, inclusive, total, ws, scheme, s);
    case OP_AND:
        return run_scan_scheme<AndU32>(in, out, n, inclusive, total, ws, scheme, s);
    case OP_OR:
        return run_scan_scheme<OrU32>(in, out, n, inclusive, total, ws, scheme, s);
    case OP_PROD:
        if (dtype == DT_FLOAT32)
            return run_scan_scheme<MulF32>(in, out, n, inclusive, total, ws, scheme, s);
        return run_scan_scheme<MulU32>(in, out, n, inclusive, total, ws, scheme, s);
    case OP_AFFINE:
        return run_scan_scheme<AffU32>(in, out, n, inclusive, total, ws, scheme, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ls
