// ls_device.hpp -- device building blocks of libscan for gfx950 (CDNA4, wave64).
//
// Lane level: a 64-lane inclusive scan in six cross-lane steps on DPP (data
// parallel primitives), no LDS and no barrier.  It is the window-doubling scan of
// the Hillis-Steele section of the parallel prefix scan page (geek-doc.cn, 二),
// applied to the lanes of a wavefront as that page's section 五 does for the 32
// lanes of a warp, with the guard "only lanes at or above the stride add": a lane
// whose source is out of range receives the operator identity.  Six steps cover
// 64 lanes where the page's warp needs five for 32.
//
// Tile level: each thread holds CHUNKS runs of 4 consecutive elements (one
// 128-bit word each).  A tile is scanned as: serial scan inside each run, wave
// scan of the run totals, a scan of the per-(run, wave) totals through LDS, and
// a carry from earlier tiles -- the "scan inside, scan the totals, add the
// offset" composition of the page's section 四, arranged so that every global
// access is a coalesced 128-bit load or store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ls {

// ---------------------------------------------------------------- operators
// Every combine in the library is written apply(earlier, later).  For the float
// max and min that order matters on ties (the later element wins), and keeping it
// everywhere makes the result independent of how the work is split.
// `commutative` says whether apply(a, b) and apply(b, a) give the same bits; a
// reduction may regroup elements out of order only when it does (float sums and
// products are commutative, if not associative).

struct SumU32 {
    using T = uint32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 0u; }
    static __device__ __forceinline__ T apply(T a, T b) { return a + b; }
};
struct XorU32 {
    using T = uint32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 0u; }
    static __device__ __forceinline__ T apply(T a, T b) { return a ^ b; }
};
struct MaxU32 {
    using T = uint32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 0u; }
    static __device__ __forceinline__ T apply(T a, T b) { return a > b ? a : b; }
};
struct MaxI32 {
    using T = int32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return INT32_MIN; }
    static __device__ __forceinline__ T apply(T a, T b) { return a > b ? a : b; }
};
struct SumF32 {
    using T = float;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 0.0f; }
    static __device__ __forceinline__ T apply(T a, T b) { return a + b; }
};
struct MaxF32 {
    using T = float;
    static constexpr bool commutative = false;
    static __device__ __forceinline__ T identity() { return -__builtin_inff(); }
    static __device__ __forceinline__ T apply(T a, T b) { return a > b ? a : b; }
};
// min keeps the later element on ties, like max.
struct MinU32 {
    using T = uint32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 0xffffffffu; }
    static __device__ __forceinline__ T apply(T a, T b) { return a < b ? a : b; }
};
struct MinI32 {
    using T = int32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return INT32_MAX; }
    static __device__ __forceinline__ T apply(T a, T b) { return a < b ? a : b; }
};
struct MinF32 {
    using T = float;
    static constexpr bool commutative = false;
    static __device__ __forceinline__ T identity() { return __builtin_inff(); }
    static __device__ __forceinline__ T apply(T a, T b) { return a < b ? a : b; }
};
struct AndU32 {
    using T = uint32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 0xffffffffu; }
    static __device__ __forceinline__ T apply(T a, T b) { return a & b; }
};
struct OrU32 {
    using T = uint32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 0u; }
    static __device__ __forceinline__ T apply(T a, T b) { return a | b; }
};
// Product: wraps modulo 2^32 for int32 and uint32 (same low bits).
struct MulU32 {
    using T = uint32_t;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 1u; }
    static __device__ __forceinline__ T apply(T a, T b) { return a * b; }
};
struct MulF32 {
    using T = float;
    static constexpr bool commutative = true;
    static __device__ __forceinline__ T identity() { return 1.0f; }
    static __device__ __forceinline__ T apply(T a, T b) { return a * b; }
};
// Composition of affine maps v -> a v + b (mod 2^16), packed (a << 16) | b: the
// 2x2 matrix [[a, b], [0, 1]].  The earlier map is applied first, so
// apply(earlier, later) is the map v -> a2 (a1 v + b1) + b2.  Not commutative: a
// scan under it checks that every combine keeps its left-right order.
struct AffU32 {
    using T = uint32_t;
    static constexpr bool commutative = false;
    static __device__ __forceinline__ T identity() { return 0x00010000u; }
    static __device__ __forceinline__ T apply(T e, T l)
    {
        const uint32_t a1 = e >> 16, b1 = e & 0xffffu, a2 = l >> 16, b2 = l & 0xffffu;
        return (((a2 * a1) & 0xffffu) << 16) | ((a2 * b1 + b2) & 0xffffu);
    }
};

template <class T>
__device__ __forceinline__ uint32_t to_bits(T v) { return __builtin_bit_cast(uint32_t, v); }
template <class T>
__device__ __forceinline__ T from_bits(uint32_t b) { return __builtin_bit_cast(T, b); }

// ---------------------------------------------------------------- DPP lane moves
// DPP control words (GFX9 encoding, valid on gfx950).
enum : int {
    DPP_ROW_SHR1 = 0x111,
    DPP_ROW_SHR2 = 0x112,
    DPP_ROW_SHR4 = 0x114,
    DPP_ROW_SHR8 = 0x118,
    DPP_WAVE_SHR1 = 0x138,
    DPP_ROW_BCAST15 = 0x142,
    DPP_ROW_BCAST31 = 0x143,
};

// Lanes whose DPP source is invalid, or whose row is masked off, return `old`.
template <int CTRL, int ROW_MASK, class T>
__device__ __forceinline__ T dpp_move(T old, T v)
{
    int r = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old), __builtin_bit_cast(int, v),
                                        CTRL, ROW_MASK, 0xf, false);
    return __builtin_bit_cast(T, r);
}

// Inclusive scan inside each row of 16 lanes (four steps: strides 1, 2, 4, 8).
template <class Op>
__device__ __forceinline__ typename Op::T row16_inclusive_scan(typename Op::T v)
{
    using T = typename Op::T;
    const T id = Op::identity();
    v = Op::apply(dpp_move<DPP_ROW_SHR1, 0xf>(id, v), v);
    v = Op::apply(dpp_move<DPP_ROW_SHR2, 0xf>(id, v), v);
    v = Op::apply(dpp_move<DPP_ROW_SHR4, 0xf>(id, v), v);
    v = Op::apply(dpp_move<DPP_ROW_SHR8, 0xf>(id, v), v);
    return v;
}

// Inclusive scan over all 64 lanes: the row scan, then lane 15 of rows 0 and 2
// is added into rows 1 and 3, then lane 31 into rows 2 and 3.
template <class Op>
__device__ __forceinline__ typename Op::T wave_inclusive_scan(typename Op::T v)
{
    using T = typename Op::T;
    const T id = Op::identity();
    v = row16_inclusive_scan<Op>(v);
    v = Op::apply(dpp_move<DPP_ROW_BCAST15, 0xa>(id, v), v);
    v = Op::apply(dpp_move<DPP_ROW_BCAST31, 0xc>(id, v), v);
    return v;
}

// Exclusive value from an inclusive one: shift up one lane, lane 0 gets identity.
template <class Op>
__device__ __forceinline__ typename Op::T wave_shift_up(typename Op::T incl)
{
    return dpp_move<DPP_WAVE_SHR1, 0xf>(Op::identity(), incl);
}

// The same inside rows of 16: lane 0 of each row gets identity.
template <class Op>
__device__ __forceinline__ typename Op::T row16_shift_up(typename Op::T incl)
{
    return dpp_move<DPP_ROW_SHR1, 0xf>(Op::identity(), incl);
}

template <class T>
__device__ __forceinline__ T read_lane(T v, int lane)
{
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------------- tile I/O
// A run of 4 consecutive 32-bit elements.
template <class T>
struct Run4 {
    T v[4];
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resources: a per-tile (base, byte count) window in scalar registers.
// Loads past the byte count return 0 and stores past it are dropped by the
// hardware, so a ragged tail needs no per-element branches; offsets are a lane
// offset in a VGPR plus a per-run constant in an SGPR.  Word 3 selects raw
// 32-bit dword access for the GFX9-family descriptor layout.
constexpr int BUF_DWORD3 = 0x00020000;
constexpr int CACHE_NT = 2;  // streaming (non-temporal) policy for data read or written once
#ifndef LS_STORE_POLICY
#define LS_STORE_POLICY 2
#endif
constexpr int STORE_POLICY = LS_STORE_POLICY;  // cache policy of the output stores

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), BUF_DWORD3);
}

// One 128-bit access (base and offsets 16-byte aligned).  The range check of a
// raw buffer access applies to each 32-bit word, so a run that straddles the end
// of the window returns its in-range words and 0 for the rest.
template <class T>
__device__ __forceinline__ Run4<T> load_run_x4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff)
{
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, CACHE_NT);
    Run4<T> r;
    r.v[0] = from_bits<T>(w.x);
    r.v[1] = from_bits<T>(w.y);
    r.v[2] = from_bits<T>(w.z);
    r.v[3] = from_bits<T>(w.w);
    return r;
}

// Four 32-bit accesses: any 4-byte alignment; each element range-checked alone,
// elements past the window read as 0.
template <class T>
__device__ __forceinline__ Run4<T> load_run_x1(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff)
{
    Run4<T> r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r.v[k] = from_bits<T>(__builtin_amdgcn_raw_buffer_load_b32(rs, voff + 4 * k, soff, CACHE_NT));
    return r;
}

// A store of more than 64 bits reads its data registers after it issues, so a
// VALU write to those registers right behind it needs a wait state.  The
// compiler inserts that wait only when the store's soffset operand is not a
// register; with the run offset in an SGPR soffset it let the next instruction
// overwrite the first data register, and gfx950 then stored the new value in
// some tiles (measured: one element per run, varying from run to run).  So the
// whole offset goes into voffset and soffset is the constant 0; tests/
// test_codegen.py checks that no 128-bit buffer store takes a register soffset.
template <class T>
__device__ __forceinline__ void store_run_x4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                             const Run4<T>& r)
{
    u32x4 w;
    w.x = to_bits(r.v[0]);
    w.y = to_bits(r.v[1]);
    w.z = to_bits(r.v[2]);
    w.w = to_bits(r.v[3]);
    __builtin_amdgcn_raw_buffer_store_b128(w, rs, voff + soff, 0, STORE_POLICY);
}

template <class T>
__device__ __forceinline__ void store_run_x1(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                             const Run4<T>& r)
{
#pragma unroll
    for (int k = 0; k < 4; ++k)
        __builtin_amdgcn_raw_buffer_store_b32(to_bits(r.v[k]), rs, voff + soff + 4 * k, 0, STORE_POLICY);  // see store_run_x4
}

// Element-wise global access with an explicit range check (row kernels).
template <class T, bool VEC>
__device__ __forceinline__ Run4<T> load_run(const T* __restrict__ p, int64_t idx, int64_t n, T fill)
{
    Run4<T> r;
    if (idx + 4 <= n) {
        if constexpr (VEC) {
            const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + idx));
            r.v[0] = from_bits<T>(w.x);
            r.v[1] = from_bits<T>(w.y);
            r.v[2] = from_bits<T>(w.z);
            r.v[3] = from_bits<T>(w.w);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                r.v[k] = p[idx + k];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            r.v[k] = (idx + k < n) ? p[idx + k] : fill;
    }
    return r;
}

template <class T, bool VEC>
__device__ __forceinline__ void store_run(T* __restrict__ p, int64_t idx, int64_t n, const Run4<T>& r)
{
    if (idx + 4 <= n) {
        if constexpr (VEC) {
            u32x4 w;
            w.x = to_bits(r.v[0]);
            w.y = to_bits(r.v[1]);
            w.z = to_bits(r.v[2]);
            w.w = to_bits(r.v[3]);
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p + idx));
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                p[idx + k] = r.v[k];
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (idx + k < n)
                p[idx + k] = r.v[k];
    }
}

// ---------------------------------------------------------------- tile status words
// One 64-bit word per tile, published and read with agent-scope atomics, so the
// flag and the value travel together and no other memory needs ordering.  Agent
// scope makes the accesses coherent across the eight XCDs (their L2s are not).
//   32-bit payload (scans): bits 63..32 = flag, bits 31..0 = value bits.
//   62-bit payload (compaction counts): bits 63..62 = flag, bits 61..0 = count.
// Each tile's word sits alone in a 256-byte slot.  Packed eight to a cache line,
// the words of neighbouring tiles are published and polled by hundreds of waves
// at once through one line; measured on MI355X that contention slowed the whole
// data stream (int32 scan of 2^28: 433 us packed, 398 us with one word per
// 256 bytes).  The cost is 256 bytes of workspace per tile.
enum : uint32_t { ST_EMPTY = 0, ST_AGGREGATE = 1, ST_PREFIX = 2 };
constexpr int STATUS_STRIDE = 32;                          // 64-bit words per tile slot
constexpr size_t STATUS_SLOT_BYTES = 8 * STATUS_STRIDE;    // workspace bytes per tile

__device__ __forceinline__ uint64_t* status_word(uint64_t* status, int64_t tile)
{
    return status + tile * STATUS_STRIDE;
}
__device__ __forceinline__ void status_store(uint64_t* p, uint64_t w)
{
    __hip_atomic_store(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t status_load(const uint64_t* p)
{
    return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded waiting: a look-back gives up after this many empty polls and records
// the fact in the workspace error word, so a defect can never hang the GPU.  In
// a correct run the wait is a few microseconds; the cap is far above that.
#ifndef LS_LOOKBACK_SPIN_LIMIT
#define LS_LOOKBACK_SPIN_LIMIT (1 << 16)
#endif
constexpr int LOOKBACK_SPIN_LIMIT = LS_LOOKBACK_SPIN_LIMIT;  // a test build sets 1 to force the give-up
constexpr uint32_t WS_ERR_LOOKBACK_TIMEOUT = 1u;

// Workspace header (first 256 bytes of every workspace).
struct WsHeader {
    uint32_t tile_counter;  // dynamic tile ids: the order in which blocks start
    uint32_t error_flags;   // WS_ERR_* bits of the last call
    uint32_t pad[62];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

// Tile id in start order: a block only ever waits for tiles that were handed to
// blocks which started before it, so every wait is for a running block.
__device__ __forceinline__ uint32_t take_tile_id(WsHeader* h)
{
    return __hip_atomic_fetch_add(&h->tile_counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void flag_error(WsHeader* h, uint32_t bits)
{
    __hip_atomic_fetch_or(&h->error_flags, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- look-back
// Status codecs: how a 64-bit status word holds (flag, value) and how values of
// a window are combined across a wave.
//
// Scan values: the operator's 32-bit element, flag in the high half.
template <class Op>
struct ScanCodec {
    using V = typename Op::T;
    static __device__ __forceinline__ uint32_t flag(uint64_t w) { return uint32_t(w >> 32); }
    static __device__ __forceinline__ V value(uint64_t w) { return from_bits<V>(uint32_t(w)); }
    static __device__ __forceinline__ uint64_t pack(uint32_t f, V v)
    {
        return (uint64_t(f) << 32) | uint64_t(to_bits(v));
    }
    static __device__ __forceinline__ V identity() { return Op::identity(); }
    static __device__ __forceinline__ V apply(V a, V b) { return Op::apply(a, b); }
    static __device__ __forceinline__ V wave_scan(V v) { return wave_inclusive_scan<Op>(v); }
    static __device__ __forceinline__ V lane(V v, int l) { return read_lane(v, l); }
    // Combine the lanes' partials in lane order (lanes below `hi` hold identity).
    static __device__ __forceinline__ V wave_reduce(V part, int /*hi*/)
    {
        return read_lane(wave_inclusive_scan<Op>(part), 63);
    }
};

// Compaction counts: 62-bit count, flag in the top two bits.  A lane's partial
// is small (a few tile counts) except on lane `hi`, whose partial includes a
// full prefix; the small ones are summed in 32 bits, the big one read whole.
struct CountCodec {
    using V = uint64_t;
    static constexpr uint64_t MASK = (uint64_t(1) << 62) - 1;
    static __device__ __forceinline__ uint32_t flag(uint64_t w) { return uint32_t(w >> 62); }
    static __device__ __forceinline__ V value(uint64_t w) { return w & MASK; }
    static __device__ __forceinline__ uint64_t pack(uint32_t f, V v) { return (uint64_t(f) << 62) | (v & MASK); }
    static __device__ __forceinline__ V identity() { return 0; }
    static __device__ __forceinline__ V apply(V a, V b) { return a + b; }
    static __device__ __forceinline__ V wave_reduce(V part, int hi)
    {
        const uint32_t small = (lane_id() > hi) ? uint32_t(part) : 0u;
        V r = read_lane(wave_inclusive_scan<SumU32>(small), 63);
        if (hi >= 0) {
            const uint32_t lo32 = __builtin_amdgcn_readlane(uint32_t(part), hi);
            const uint32_t hi32 = __builtin_amdgcn_readlane(uint32_t(part >> 32), hi);
            r += (uint64_t(hi32) << 32) | lo32;
        }
        return r;
    }
};

// Exclusive prefix of tile `tile` (>= 1), computed by one full wave from the
// tile status words.  A poll reads a window of WIDE tiles (at most 64), lane l
// holding tile last - 63 + l.  In the window, the newest tile that has published
// a full prefix ends the walk: the answer is the operator over it and every newer
// tile of the window.  Without one, the window's totals are combined and the
// window moves WIDE tiles back.  An empty word newer than the stopping tile means
// that tile has not published yet: sleep, then poll again.  The first poll reads
// only the eight nearest tiles, which settles tiles whose predecessor is already
// done.  Every status word sits in its own 256-byte slot, so a poll costs one
// coherent request per tile read: windows of 128 to 512 words per poll and
// shorter sleeps were measured slower, because the polls load the memory system
// that the tiles' data also goes through.  Narrow windows win on MI355X: the
// segmented scan and compaction poll 8 tiles at a time (measured on the plain
// scan when it still walked back, 2^28: 347-349 us against 353 for 16 and 367
// for 64, and 355-356 us for windows that double after each window without a
// full prefix, up to 32 or 64).  The plain scan now uses chased prefixes (below).
constexpr int LB_WINDOW = 64;
constexpr int LB_NEAR = 8;      // tiles read by the first, narrow poll
constexpr int LB_SLEEP = 32;    // s_sleep units (64 clocks each) between polls

template <class Codec, int WIDE = LB_WINDOW>
__device__ typename Codec::V lookback(const uint64_t* status, int64_t tile, WsHeader* hdr)
{
    static_assert(WIDE >= LB_NEAR && WIDE <= LB_WINDOW, "a wide poll reads LB_NEAR to 64 tiles");
    using V = typename Codec::V;
    const int lane = lane_id();
    auto word = [&](int64_t idx) -> uint64_t {
        return idx >= 0 ? status_load(status + idx * STATUS_STRIDE) : Codec::pack(ST_PREFIX, Codec::identity());
    };
    if constexpr (WIDE > LB_NEAR) {
        // narrow first poll: lanes 56..63 read the eight nearest tiles; the
        // other lanes stand for tiles that do not take part (identity totals).
        // With WIDE == LB_NEAR the loop's first poll reads the same words.
        const bool near = lane >= LB_WINDOW - LB_NEAR;
        const uint64_t w = near ? word(tile - LB_WINDOW + lane) : Codec::pack(ST_AGGREGATE, Codec::identity());
        const uint64_t has = __ballot(near && Codec::flag(w) == ST_PREFIX);
        const int hi = has ? 63 - __builtin_clzll(has) : -1;
        if (hi >= 0 && !__ballot(lane > hi && Codec::flag(w) == ST_EMPTY))
            return Codec::wave_reduce(lane >= hi ? Codec::value(w) : Codec::identity(), hi);
    }
    V excl = Codec::identity();
    int64_t last = tile - 1;
    int spins = 0;
    for (;;) {
        // lanes 64 - WIDE .. 63 read the WIDE newest tiles not yet combined
        const bool act = lane >= LB_WINDOW - WIDE;
        const uint64_t w = act ? word(last - (LB_WINDOW - 1) + lane) : Codec::pack(ST_AGGREGATE, Codec::identity());
        const uint64_t has = __ballot(act && Codec::flag(w) == ST_PREFIX);
        const int hi = has ? 63 - __builtin_clzll(has) : -1;
        if (__ballot(act && lane > hi && Codec::flag(w) == ST_EMPTY)) {
            if (++spins < LOOKBACK_SPIN_LIMIT) {
                __builtin_amdgcn_s_sleep(LB_SLEEP);
                continue;
            }
            if (lane == 0)
                flag_error(hdr, WS_ERR_LOOKBACK_TIMEOUT);
            return excl;  // only reached on a defect; the error word reports it
        }
        const V part = lane >= hi ? Codec::value(w) : Codec::identity();
        excl = Codec::apply(Codec::wave_reduce(part, hi), excl);  // older tiles on the left
        if (hi >= 0)
            return excl;
        last -= WIDE;
    }
}

// ---------------------------------------------------------------- chased prefixes
// The single-pass scan does not let every tile walk back on its own.  One wave
// (the one that scanned tile 0) stays resident after its tile and moves the
// "full prefix" frontier forward for everyone: it polls the status words of the
// current group of 64 tiles, takes the run of consecutive tiles that have
// published their totals, scans them across the wave, and publishes a full prefix
// for each (chase_prefixes below).  Every other tile publishes its total and then
// polls one word, its predecessor's, until that word holds a full prefix: its
// own exclusive prefix.  Only the chasing wave writes full prefixes (besides
// tile 0), so each tile's prefix is computed once and every tile sees the same
// value.
//
// Why: traced on MI355X (int32 scan of 2^28), walking tiles took 5.7 polls of
// 8 words each (about 45 status reads) to reach a published prefix, because the
// prefixes themselves waited on those walks.  Waiting on one word cuts the
// status reads per tile to a few, and the wait after the last needed load to one
// chaser cycle plus one poll.  That traffic saving lets smaller tiles pay:
// 338 us against 348 us for the scan of 2^28 (26624- against 32768-element
// tiles, each scheme at its best size).  With windows that started at the
// frontier, a chaser reading 16 or 32 words per poll could not keep up with the
// tiles (458 / 357 us), and 128 or 256 words per poll (two or four per lane) were
// slower as well (358 / 390 us).
//
// Progress: the chaser only reads totals, and a tile publishes its total without
// waiting for anything; a tile with an id is resident, because ids are taken in
// start order.  So the frontier always reaches every tile, and both loops are
// bounded like the look-back (the error word reports a cap that is hit).
constexpr int LB_WAIT_SLEEP = 8;    // s_sleep units between a tile's polls of its predecessor
constexpr int LB_CHASE_SLEEP = 2;   // between chaser polls that found nothing new

// Exclusive prefix of `tile` (>= 1): the full prefix that the chaser publishes
// in the status word of tile - 1.  Called by a whole wave; every lane reads the
// same word.
template <class Codec>
__device__ typename Codec::V wait_prefix(const uint64_t* status, int64_t tile, WsHeader* hdr)
{
    const uint64_t* p = status + (tile - 1) * STATUS_STRIDE;
    int spins = 0;
    for (;;) {
        const uint64_t w = status_load(p);
        if (__ballot(Codec::flag(w) == ST_PREFIX))
            return Codec::value(w);
        if (++spins >= LOOKBACK_SPIN_LIMIT) {
            if (lane_id() == 0)
                flag_error(hdr, WS_ERR_LOOKBACK_TIMEOUT);
            return Codec::identity();  // only reached on a defect; the error word reports it
        }
        __builtin_amdgcn_s_sleep(LB_WAIT_SLEEP);
    }
}

// Publishes the full prefix of tiles 1 .. num_tiles - 1, in order, given the
// full prefix of tile 0.  Called by one whole wave, after tile 0 is published.
// Tiles form groups of 64 aligned to tile 0, lane l standing for tile 64 G + l.
// The wave keeps the totals of the group's tiles it has seen in its lanes and
// polls only the lanes still missing; once lanes 0 .. k-1 hold totals it scans the
// group across the wave and publishes the new ones on top of the previous group's
// last full prefix.  Lane j's scan value depends on lanes 0 .. j only, through a
// tree fixed by j, so every tile's full prefix is a fixed function of the tile
// totals, whatever a poll happened to find: float results are the same bits on
// every run (MI355X, float32 sum of 2^26: one distinct result in 10 runs, against
// 10 in 10 for windows that start at the frontier, at the same speed).  A tile
// whose full prefix does not depend on earlier tiles (a segmented tile containing a
// head) may publish it itself; the wave takes such a word as that tile's total --
// its scan gives the same value there -- and does not publish it again.
template <class Codec>
__device__ void chase_prefixes(uint64_t* status, int64_t num_tiles, typename Codec::V prefix, WsHeader* hdr)
{
    using V = typename Codec::V;
    const int lane = lane_id();
    int64_t g0 = 0;                                  // first tile of the current group
    V base = Codec::identity();                      // full prefix of tile g0 - 1
    V tot = lane == 0 ? prefix : Codec::identity();  // totals of the group's tiles seen so far
    int have = 1;                                    // lanes 0 .. have-1 hold their totals
    int idle = 0;
    while (g0 + have < num_tiles) {
        const int64_t idx = g0 + lane;
        const bool want = lane >= have && idx < num_tiles;
        const uint64_t w = want ? status_load(status + idx * STATUS_STRIDE) : 0ull;
        const bool pub = want && Codec::flag(w) == ST_AGGREGATE;  // still to be published
        const bool ready = lane < have || pub || (want && Codec::flag(w) == ST_PREFIX);
        const uint64_t miss = __ballot(!ready);
        const int k = miss ? __builtin_ctzll(miss) : 64;  // lanes 0 .. k-1 now hold totals
        if (k == have) {
            if (++idle >= LOOKBACK_SPIN_LIMIT) {
                if (lane == 0)
                    flag_error(hdr, WS_ERR_LOOKBACK_TIMEOUT);
                return;  // only reached on a defect; the error word reports it
            }
            __builtin_amdgcn_s_sleep(LB_CHASE_SLEEP);
            continue;
        }
        idle = 0;
        if (lane >= have && lane < k)
            tot = Codec::value(w);
        // older on the left: base (+) totals of tiles g0 .. g0 + lane
        const V inc = Codec::apply(base, Codec::wave_scan(lane < k ? tot : Codec::identity()));
        if (lane >= have && lane < k && pub)
            status_store(status + idx * STATUS_STRIDE, Codec::pack(ST_PREFIX, inc));
        have = k;
        if (have == 64) {
            base = Codec::lane(inc, 63);
            g0 += 64;
            have = 0;
            tot = Codec::identity();
        }
    }
}

// Fixed-association variant ([Scan3] pitfall list: float addition does not
// associate, so a reproducible result needs a fixed order).  Tiles form groups
// of LB_GROUP.  Only the last tile of a group publishes a full prefix; every
// other tile publishes only its total.  Tile t's exclusive prefix is the full
// prefix of the last tile of the previous group combined with the totals of the
// earlier tiles of its own group, all in one wave in lane order (lane 0 the
// prefix, lane l the total of the group's tile l - 1).  Which words are combined,
// and how, depends only on t, never on timing, so the result is the same bits on
// every run.  The price: a tile waits for exactly those words (no adaptive walk).
constexpr int LB_GROUP = 64;

template <class Codec>
__device__ typename Codec::V lookback_grouped(const uint64_t* status, int64_t tile, WsHeader* hdr)
{
    const int lane = lane_id();
    const int64_t g0 = tile - tile % LB_GROUP;  // first tile of this tile's group
    const int before = int(tile - g0);         // tiles of the group before this one
    const bool needed = lane == 0 ? g0 > 0 : lane <= before;
    const int64_t idx = lane == 0 ? g0 - 1 : g0 + lane - 1;
    int spins = 0;
    for (;;) {
        const uint64_t w = needed ? status_load(status + idx * STATUS_STRIDE)
                                  : Codec::pack(ST_AGGREGATE, Codec::identity());
        const uint32_t f = Codec::flag(w);
        const bool ready = !needed || (lane == 0 ? f == ST_PREFIX : f != ST_EMPTY);
        if (!__ballot(!ready))
            return Codec::wave_reduce(needed ? Codec::value(w) : Codec::identity(), -1);
        if (++spins >= LOOKBACK_SPIN_LIMIT) {
            if (lane == 0)
                flag_error(hdr, WS_ERR_LOOKBACK_TIMEOUT);
            return Codec::identity();  // only reached on a defect; the error word reports it
        }
        __builtin_amdgcn_s_sleep(LB_SLEEP);
    }
}

}  // namespace ls
