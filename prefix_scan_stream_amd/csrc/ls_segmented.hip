// ls_segmented.hip -- segmented scan in one pass (gfx950).
//
// A segmented scan restarts at every segment boundary (lpnh.cn parallel scan
// overview, section 7.2).  Segments are marked by a head flag on their first
// element, or given as CSR offsets.  The scan runs the single-pass machinery of
// the plain scan on (head, value) pairs under the lifted operator
//     (h1, v1) then (h2, v2)  =  (h1 | h2,  h2 ? v2 : v1 (+) v2),
// which is associative but not commutative: a head in the later span cuts the
// earlier value off.  Per tile (16384 elements, 512 threads x 8 runs of 4):
//   1. take a tile id in start order, load the values (128-bit loads) and the
//      head bits of every run (flag bytes, or a head bitmap that the tile builds
//      in LDS from its own range of the offsets);
//   2. scan each run in registers, restarting at heads; scan the run pairs across
//      the wave (DPP on the value and the head bit), the (run, wave) pairs in LDS;
//   3. the first wave publishes the tile's pair and takes its carry from the
//      chased prefixes (ls_device.hpp): the full prefix of the previous tile.  A
//      tile that contains a head publishes its full prefix at once (nothing before
//      the head can reach past it), the others their totals, which the chasing
//      wave turns into full prefixes in an order fixed by the tile index, so float
//      sums repeat bit for bit.  A tile whose first element is a head needs no
//      carry.  Head tiles publishing at once keep most waits short: int32 sums of
//      2^26 with head flags / CSR offsets 106 / 98 us, against 109-110 / 102-103 us
//      when every tile walked back (and 113-115 / 109-110 us when head tiles also
//      waited for the chasing wave);
//   4. every element combines the carry into its run with its own in-run value,
//      unless a head in the run lies at or before it.
// Elements past n read as 0 and sit after every valid element, as in the plain
// scan.  HBM traffic: n*4 read + n*4 written, plus n flag bytes or the offsets.
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

// 8-wave blocks of 8 runs per thread: 16384-element tiles at about 83 VGPRs, two
// blocks per CU.  A (value, head) pair doubles the scan's registers, so the tile
// is half the plain scan's.  int32 sums of 2^26 with head flags / CSR offsets:
// 109-110 / 102 us, against 116-117 / 107 us for 4-wave blocks of 16 runs (the
// same tile, 160 VGPRs, three blocks per CU), 111-112 / 102-103 us for 10 or 12
// runs, and 131 us for 16 runs in 8-wave blocks (one block per CU).
#ifndef LS_SG_BLOCK
#define LS_SG_BLOCK 512
#endif
#ifndef LS_SG_CHUNKS
#define LS_SG_CHUNKS 8
#endif
constexpr int SG_BLOCK = LS_SG_BLOCK;
constexpr int SG_WAVES = SG_BLOCK / 64;
constexpr int SG_CHUNKS = LS_SG_CHUNKS;
constexpr int SG_TILE = SG_BLOCK * SG_CHUNKS * 4;  // 16384 elements

enum SegSource : int { SEG_FLAGS = 0, SEG_OFFSETS = 1 };

// A (value, head) pair: head != 0 when a segment starts inside the span the
// value covers (the value then covers only the part from the last head on).
template <class Op>
struct SegPair {
    typename Op::T v;
    uint32_t h;
};

template <class Op>
__device__ __forceinline__ SegPair<Op> seg_identity()
{
    return {Op::identity(), 0u};
}

// earlier then later
template <class Op>
__device__ __forceinline__ SegPair<Op> seg_apply(SegPair<Op> a, SegPair<Op> b)
{
    return {b.h ? b.v : Op::apply(a.v, b.v), a.h | b.h};
}

template <int CTRL, int ROW_MASK, class Op>
__device__ __forceinline__ SegPair<Op> seg_dpp(SegPair<Op> old, SegPair<Op> p)
{
    return {dpp_move<CTRL, ROW_MASK>(old.v, p.v), dpp_move<CTRL, ROW_MASK>(old.h, p.h)};
}

// The wave scan of the plain scan (rows of 16 by row_shr, then the row
// broadcasts), on pairs.
template <class Op>
__device__ __forceinline__ SegPair<Op> seg_wave_inclusive_scan(SegPair<Op> p)
{
    const SegPair<Op> id = seg_identity<Op>();
    p = seg_apply<Op>(seg_dpp<DPP_ROW_SHR1, 0xf>(id, p), p);
    p = seg_apply<Op>(seg_dpp<DPP_ROW_SHR2, 0xf>(id, p), p);
    p = seg_apply<Op>(seg_dpp<DPP_ROW_SHR4, 0xf>(id, p), p);
    p = seg_apply<Op>(seg_dpp<DPP_ROW_SHR8, 0xf>(id, p), p);
    p = seg_apply<Op>(seg_dpp<DPP_ROW_BCAST15, 0xa>(id, p), p);
    p = seg_apply<Op>(seg_dpp<DPP_ROW_BCAST31, 0xc>(id, p), p);
    return p;
}

template <class Op>
__device__ __forceinline__ SegPair<Op> seg_wave_shift_up(SegPair<Op> incl)
{
    return seg_dpp<DPP_WAVE_SHR1, 0xf>(seg_identity<Op>(), incl);
}

template <class Op>
__device__ __forceinline__ SegPair<Op> seg_read_lane(SegPair<Op> p, int lane)
{
    return {read_lane(p.v, lane), read_lane(p.h, lane)};
}

// Status word of a tile: bits 63..62 status flag, bit 61 head, bits 60..32 the
// call's epoch (29 bits), bits 31..0 value.
template <class Op>
struct SegCodec {
    using V = SegPair<Op>;
    static constexpr uint32_t EPOCH_MASK = (1u << 29) - 1u;
    static __device__ __forceinline__ uint32_t flag(uint64_t w, uint32_t ep)
    {
        return ((uint32_t(w >> 32) & EPOCH_MASK) == (ep & EPOCH_MASK)) ? uint32_t(w >> 62) : ST_EMPTY;
    }
    static __device__ __forceinline__ V value(uint64_t w)
    {
        return {from_bits<typename Op::T>(uint32_t(w)), uint32_t(w >> 61) & 1u};
    }
    static __device__ __forceinline__ uint64_t pack(uint32_t f, V p, uint32_t ep)
    {
        return (uint64_t(f) << 62) | (uint64_t(p.h ? 1u : 0u) << 61) | (uint64_t(ep & EPOCH_MASK) << 32) |
               uint64_t(to_bits(p.v));
    }
    static __device__ __forceinline__ V identity() { return seg_identity<Op>(); }
    static __device__ __forceinline__ V apply(V a, V b) { return seg_apply<Op>(a, b); }
    // a tile that contains a head publishes its full prefix itself
    static __device__ __forceinline__ bool self_published(V p) { return p.h != 0u; }
    static __device__ __forceinline__ V wave_reduce(V part, int /*hi*/)
    {
        return seg_read_lane<Op>(seg_wave_inclusive_scan<Op>(part), 63);
    }
    static __device__ __forceinline__ V wave_scan(V v) { return seg_wave_inclusive_scan<Op>(v); }
    static __device__ __forceinline__ V lane(V v, int l) { return seg_read_lane<Op>(v, l); }
};

template <class Op, bool INCLUSIVE, bool VEC, int SRC>
__global__ __launch_bounds__(SG_BLOCK) void seg_scan_kernel(const typename Op::T* __restrict__ in,
                                                            typename Op::T* __restrict__ out, int64_t n,
                                                            int64_t num_tiles, const uint8_t* __restrict__ heads,
                                                            bool heads4, const int64_t* __restrict__ offsets,
                                                            int64_t nseg, WsHeader* hdr, uint64_t* status,
                                                            typename Op::T* total)
{
    using T = typename Op::T;
    using P = SegPair<Op>;
    using Codec = SegCodec<Op>;
    constexpr int PARTS = SG_CHUNKS * SG_WAVES;
    constexpr int PPL = (PARTS + 63) / 64;  // (run, wave) pairs per lane in their scan
    constexpr uint32_t RUN_STRIDE = SG_BLOCK * 16u;
    static_assert(PARTS % PPL == 0 && PARTS / PPL <= 64, "the (run, wave) pairs are scanned by one wave");
    __shared__ T s_pv[PARTS];
    __shared__ uint32_t s_ph[PARTS];
    __shared__ uint64_t s_ticket;
    __shared__ int64_t s_k0;
    __shared__ uint32_t s_bits[SRC == SEG_OFFSETS ? SG_TILE / 32 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const T id = Op::identity();

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
    const int64_t tile = ticket_tile(ticket);
    const uint32_t ep = ticket_epoch(ticket);
    if (tile >= num_tiles)
        return;  // uniform over the block: a workspace that was not initialised
    const int64_t tbase = tile * SG_TILE;
    const int64_t rem = n - tbase;
    const uint32_t valid = rem < SG_TILE ? uint32_t(rem) : uint32_t(SG_TILE);
    const bool full = valid == SG_TILE;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tbase, valid * 4u);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + tbase, valid * 4u);
    const uint32_t voff = uint32_t(tid) * 16u;

    // 1. values and head bits (bit k of hb[j]: element k of run j starts a segment)
    Run4<T> r[SG_CHUNKS];
#pragma unroll
    for (int j = 0; j < SG_CHUNKS; ++j)
        r[j] = VEC ? load_run_x4<T>(rin, voff, j * RUN_STRIDE) : load_run_x1<T>(rin, voff, j * RUN_STRIDE);
    uint32_t hb[SG_CHUNKS];
    if constexpr (SRC == SEG_OFFSETS) {
        for (int i = tid; i < SG_TILE / 32; i += SG_BLOCK)
            s_bits[i] = 0u;
        if (tid == 0) {
            // first k in [0, nseg] with offsets[k] >= tbase (offsets non-decreasing)
            int64_t lo = 0, hi = nseg;
            while (lo < hi) {
                const int64_t mid = lo + (hi - lo) / 2;
                if (offsets[mid] < tbase)
                    lo = mid + 1;
                else
                    hi = mid;
            }
            s_k0 = lo;
        }
        __syncthreads();
        for (int64_t k = s_k0 + tid; k < nseg; k += SG_BLOCK) {
            const int64_t o = offsets[k] - tbase;
            if (o >= int64_t(valid))
                break;
            if (o >= 0)  // malformed (unsorted) offsets may fall before the tile: ignore them
                atomicOr(&s_bits[o >> 5], 1u << (o & 31));
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < SG_CHUNKS; ++j) {
            const uint32_t e0 = 4u * uint32_t(j * SG_BLOCK + tid);  // 4-aligned: one word
            hb[j] = (s_bits[e0 >> 5] >> (e0 & 31)) & 0xfu;
        }
    } else {
        const __amdgpu_buffer_rsrc_t rfl = make_rsrc(heads + tbase, valid);
#pragma unroll
        for (int j = 0; j < SG_CHUNKS; ++j) {
            const uint32_t b0 = 4u * uint32_t(j * SG_BLOCK + tid);
            uint32_t w;
            // a dword straddling the end of the range reads as 0 as a whole, so the
            // run holding a ragged tile's last flags (and unaligned arrays) read bytes
            if (heads4 && (b0 + 4u <= valid || b0 >= valid)) {
                w = __builtin_amdgcn_raw_buffer_load_b32(rfl, b0, 0, CACHE_NT);
            } else {
                w = 0;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    w |= uint32_t(__builtin_amdgcn_raw_buffer_load_b8(rfl, b0 + k, 0, CACHE_NT)) << (8 * k);
            }
            uint32_t m = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k)
                m |= (((w >> (8 * k)) & 0xffu) != 0u ? 1u : 0u) << k;
            hb[j] = m;
        }
    }
    if (tile == 0 && tid == 0)
        hb[0] |= 1u;  // element 0 always starts a segment

    // 2. run scans restarting at heads; wave scan of the run pairs
    uint32_t wexh = 0;  // bit j: a head in an earlier run of this run's wave row
    T wexv[SG_CHUNKS];
#pragma unroll
    for (int j = 0; j < SG_CHUNKS; ++j) {
#pragma unroll
        for (int k = 1; k < 4; ++k)
            r[j].v[k] = ((hb[j] >> k) & 1u) ? r[j].v[k] : Op::apply(r[j].v[k - 1], r[j].v[k]);
        const P inc = seg_wave_inclusive_scan<Op>(P{r[j].v[3], hb[j] != 0u ? 1u : 0u});
        const P ex = seg_wave_shift_up<Op>(inc);
        wexv[j] = ex.v;
        wexh |= (ex.h ? 1u : 0u) << j;
        if (lane == 63) {
            s_pv[j * SG_WAVES + wave] = inc.v;
            s_ph[j * SG_WAVES + wave] = inc.h;
        }
    }
    __syncthreads();

    // 3. wave 0: scan the (run, wave) pairs, publish, take the carry
    P agg0 = seg_identity<Op>();  // tile 0's pair: where the chasing wave starts
    if (wave == 0) {
        // lane l holds pairs PPL l .. PPL l + PPL - 1, combined in element order
        P pv[PPL];
        P part = seg_identity<Op>();
#pragma unroll
        for (int q = 0; q < PPL; ++q) {
            const int i = PPL * lane + q;
            pv[q] = i < PARTS ? P{s_pv[i], s_ph[i]} : seg_identity<Op>();
            part = seg_apply<Op>(part, pv[q]);
        }
        const P inc = seg_wave_inclusive_scan<Op>(part);
        const P exc = seg_wave_shift_up<Op>(inc);
        const P agg = seg_read_lane<Op>(inc, 63);
        P carry = seg_identity<Op>();
        // every tile publishes its total; tile 0 and tiles containing a head also
        // their full prefix, which then does not depend on earlier tiles
        if (lane == 0) {
            status_store(total_word(status, tile), Codec::pack(ST_AGGREGATE, agg, ep));
            if (tile == 0 || agg.h)
                status_store(status_word(status, tile), Codec::pack(ST_PREFIX, agg, ep));
        }
        if (tile == 0) {
            agg0 = agg;
        } else {
            const bool first_is_head = __builtin_amdgcn_readfirstlane(hb[0] & 1u) != 0u;
            if (!first_is_head && !wait_prefix<Codec>(status, tile, ep, carry, WAIT_LIMIT_TICKS)) {
                if (lane == 0)
                    flag_error(hdr, WS_ERR_WAIT_TIMEOUT);  // only on a defect: tickets make every wait finite
            }
        }
        P e = seg_apply<Op>(carry, exc);
#pragma unroll
        for (int q = 0; q < PPL; ++q) {
            const int i = PPL * lane + q;
            if (i < PARTS) {
                s_pv[i] = e.v;
                s_ph[i] = e.h;
            }
            e = seg_apply<Op>(e, pv[q]);
        }
    }
    __syncthreads();

    // 4. finish and store; the thread holding element n-1 writes the total (the
    // inclusive value of element n-1: the last segment's reduction)
    const int64_t last_local = (tile == num_tiles - 1) ? int64_t(valid) - 1 : -1;
#pragma unroll
    for (int j = 0; j < SG_CHUNKS; ++j) {
        const P sp = {s_pv[j * SG_WAVES + wave], s_ph[j * SG_WAVES + wave]};
        const T cv = seg_apply<Op>(sp, P{wexv[j], (wexh >> j) & 1u}).v;  // flows into element 0 of the run
        T incl[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            incl[k] = (hb[j] & ((2u << k) - 1u)) ? r[j].v[k] : Op::apply(cv, r[j].v[k]);
        Run4<T> o;
        if constexpr (INCLUSIVE) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o.v[k] = incl[k];
        } else {
            o.v[0] = (hb[j] & 1u) ? id : cv;
#pragma unroll
            for (int k = 1; k < 4; ++k)
                o.v[k] = ((hb[j] >> k) & 1u) ? id : incl[k - 1];
        }
        if (VEC && full)
            store_run_x4<T>(rout, voff, j * RUN_STRIDE, o);
        else
            store_run_x1<T>(rout, voff, j * RUN_STRIDE, o);
        if (total != nullptr) {
            const int64_t kk = last_local - 4 * int64_t(j * SG_BLOCK + tid);
            if (kk >= 0 && kk < 4) {
                T v = incl[0];  // select, not index: keeps the tile in registers
#pragma unroll
                for (int k = 1; k < 4; ++k)
                    v = (kk == k) ? incl[k] : v;
                *total = v;
            }
        }
    }
    // 5. tile 0's first wave, its own tile written, publishes the later tiles' full
    // prefixes (it returns once the last tile's is out)
    if (tile == 0 && wave == 0)
        chase_prefixes<Codec>(status, num_tiles, agg0, ep);
}

// ------------------------------------------------------------------ host side

static int64_t sg_tiles(int64_t n) { return (n + SG_TILE - 1) / SG_TILE; }

size_t segmented_workspace_bytes(int64_t n)
{
    const int64_t t = sg_tiles(n);
    const size_t bytes = sizeof(WsHeader) + size_t(t < 1 ? 1 : t) * STATUS_SLOT_BYTES;
    return (bytes + 255) & ~size_t(255);
}

template <class Op>
__global__ void seg_store_identity_kernel(typename Op::T* total)
{
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *total = Op::identity();
}

template <class Op, int SRC>
static hipError_t run_segmented(const void* in, void* out, int64_t n, bool excl, const uint8_t* heads,
                                const int64_t* offsets, int64_t nseg, void* total, void* ws, hipStream_t s)
{
    using T = typename Op::T;
    if (n == 0) {  // no segment: the total is the identity; nothing else to enqueue
        if (total == nullptr)
            return hipSuccess;
        hipLaunchKernelGGL(seg_store_identity_kernel<Op>, dim3(1), dim3(64), 0, s, reinterpret_cast<T*>(total));
        return hipGetLastError();
    }
    const int64_t tiles = sg_tiles(n);
    auto* hdr = reinterpret_cast<WsHeader*>(ws);
    auto* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    const bool heads4 = (reinterpret_cast<uintptr_t>(heads) & 3) == 0;
    const T* pin = reinterpret_cast<const T*>(in);
    T* pout = reinterpret_cast<T*>(out);
    T* ptot = reinterpret_cast<T*>(total);
    const dim3 grid(static_cast<uint32_t>(tiles)), block(SG_BLOCK);
#define LS_SG(INCL, V)                                                                                   \
    hipLaunchKernelGGL((seg_scan_kernel<Op, INCL, V, SRC>), grid, block, 0, s, pin, pout, n, tiles, heads, \
                       heads4, offsets, nseg, hdr, status, ptot)
    if (!excl) {
        if (vec) LS_SG(true, true); else LS_SG(true, false);
    } else {
        if (vec) LS_SG(false, true); else LS_SG(false, false);
    }
#undef LS_SG
    return hipGetLastError();
}

template <int SRC>
static hipError_t dispatch_segmented(const void* in, void* out, int64_t n, int dtype, int op, bool excl,
                                     const uint8_t* heads, const int64_t* offsets, int64_t nseg,
                                     void* total, void* ws, hipStream_t s)
{
#define LS_RUN(OPT) return run_segmented<OPT, SRC>(in, out, n, excl, heads, offsets, nseg, total, ws, s)
    switch (op) {
    case OP_SUM: if (dtype == DT_FLOAT32) LS_RUN(SumF32); LS_RUN(SumU32);
    case OP_XOR: LS_RUN(XorU32);
    case OP_MAX:
        if (dtype == DT_INT32) LS_RUN(MaxI32);
        if (dtype == DT_UINT32) LS_RUN(MaxU32);
        LS_RUN(MaxF32);
    case OP_MIN:
        if (dtype == DT_INT32) LS_RUN(MinI32);
        if (dtype == DT_UINT32) LS_RUN(MinU32);
        LS_RUN(MinF32);
    case OP_AND: LS_RUN(AndU32);
    case OP_OR: LS_RUN(OrU32);
    case OP_PROD: if (dtype == DT_FLOAT32) LS_RUN(MulF32); LS_RUN(MulU32);
    case OP_AFFINE: LS_RUN(AffU32);
    }
#undef LS_RUN
    return hipErrorInvalidValue;
}

hipError_t launch_segmented(const void* in, void* out, int64_t n, int dtype, int op, bool excl,
                            const uint8_t* heads, const int64_t* offsets, int64_t nseg, void* total,
                            void* ws, hipStream_t s)
{
    if (offsets != nullptr)
        return dispatch_segmented<SEG_OFFSETS>(in, out, n, dtype, op, excl, nullptr, offsets, nseg, total, ws, s);
    return dispatch_segmented<SEG_FLAGS>(in, out, n, dtype, op, excl, heads, nullptr, 0, total, ws, s);
}

}  // namespace ls
