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
// Every word also carries the epoch of the call that wrote it (below); a word
// whose epoch is not the reader's reads as empty, so words left by earlier calls
// never need clearing.
//   32-bit payload (scans): bits 63..62 flag, 61..32 epoch (30 bits), 31..0 value.
//   36-bit payload (compaction counts): 63..62 flag, 61..58 count bits 35..32,
//     57..32 epoch (26 bits), 31..0 count bits 31..0.
// The segmented scan's words add a head bit (ls_segmented.hip).  Every format keeps
// its epoch's low bits from bit 32 up, so a word of one format never reads as
// current to a reader of another at a later epoch.
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

// Bounded waiting, on the wall clock (100 MHz on MI355X).  In a correct run a wait
// for another tile lasts microseconds.
//   A wait that can only give up (ticket tiles, and the chasing wave) does so
//   after about one second without progress and records it in the workspace
//   error word, so a defect can never hang the GPU.
//   A wait with a fallback (block-index tiles) stops after about a millisecond
//   and computes what it waited for itself: the tile it waits for may belong to
//   a block that is not resident yet.
// A test build sets both limits to 0: every wait then stops at its first empty poll.
#ifndef LS_WAIT_LIMIT_TICKS
#define LS_WAIT_LIMIT_TICKS 100000000ull
#endif
#ifndef LS_FALLBACK_TICKS
#define LS_FALLBACK_TICKS 100000ull
#endif
constexpr uint64_t WAIT_LIMIT_TICKS = LS_WAIT_LIMIT_TICKS;
constexpr uint64_t FALLBACK_TICKS = LS_FALLBACK_TICKS;
constexpr uint32_t WS_ERR_WAIT_TIMEOUT = 1u;  // a wait gave up: that call's output is incomplete
constexpr uint32_t WS_ERR_BAD_TICKET = 2u;    // a tile id past the call's tiles (workspace not initialised,
                                              // or shared by calls that overlap)

// Start of a wait, and whether its time is up (read only after an empty poll).
__device__ __forceinline__ uint64_t wait_start() { return wall_clock64(); }
__device__ __forceinline__ bool wait_expired(uint64_t start, uint64_t limit = WAIT_LIMIT_TICKS)
{
    return uint64_t(wall_clock64()) - start >= limit;
}

// Workspace header (first 256 bytes of every workspace).  A workspace starts
// zero-filled (ls_workspace_init) and every call leaves it ready for the next:
// the epoch advanced, the counters back at 0.  Calls need no clearing launch.
struct WsHeader {
    uint64_t ticket;       // bits 63..32: the current call's epoch; bits 31..0: tickets handed out so far
    uint32_t error_flags;  // WS_ERR_* bits, kept until the workspace is initialised again
    uint32_t started;      // the compaction: blocks that have read the current epoch
    uint32_t pad[60];
};
static_assert(sizeof(WsHeader) == 256, "workspace header is 256 bytes");

__device__ __forceinline__ uint32_t ticket_tile(uint64_t t) { return uint32_t(t); }
__device__ __forceinline__ uint32_t ticket_epoch(uint64_t t) { return uint32_t(t >> 32); }

// The next call on this workspace runs under the next epoch, with no tickets out.
__device__ __forceinline__ void start_next_epoch(WsHeader* h, uint32_t epoch)
{
    __hip_atomic_store(&h->ticket, uint64_t(epoch + 1u) << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Two ways of giving tiles to blocks.
//
// Tickets (segmented scans, the fixed-order and the affine-map scans): a block
// takes the next tile id from a counter in the order blocks start, so a block only
// ever waits for tiles that were handed to blocks which started before it: every
// wait is for a running block.  The ticket carries the call's epoch in its high
// half; the block that takes the call's last tile (all tickets are then out)
// starts the next epoch.
__device__ __forceinline__ uint64_t take_ticket(WsHeader* h)
{
    return __hip_atomic_fetch_add(&h->ticket, uint64_t(1), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block index (the plain single-pass scan and the compaction): tile = the block's
// index (the compaction's persistent blocks: every G-th tile from it), which
// costs no atomic at the start of a block (one device-scope atomic on one address
// serializes at about 12 ns on MI355X, which is most of the gap between a tiled
// copy and the scan).  Without tickets, a tile may wait for a tile whose block
// has not been dispatched, so every such wait has a fallback that needs no other
// block: after FALLBACK_TICKS the waiting tile computes what it waits for from
// the input itself (replay_prefix below; the compaction's recounting look-back).
// The call's epoch is read from the header at each block's start.  The block
// that finishes the call's last tile starts the next epoch once no block can
// still read the old one.  In the scan: when its prefix came from the chasing
// wave, that wave had seen the totals of every earlier tile, each written by its
// own block after reading the epoch, so every block had started; when it
// computed its prefix itself, it first waits until every earlier tile's own block
// has published its total (await_totals).  The compaction counts started blocks
// (mark_started, end_call below).
__device__ __forceinline__ uint32_t read_epoch(WsHeader* h)
{
    return ticket_epoch(__hip_atomic_load(&h->ticket, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// await_totals waits for blocks that will certainly run (each starts as soon as
// others finish); its limit only guards against defects.
constexpr uint64_t AWAIT_LIMIT_TICKS = 1000000000ull;  // about 10 s

__device__ __forceinline__ void flag_error(WsHeader* h, uint32_t bits);

// The compaction's walking look-back does not tell the last tile whether every
// block has read the epoch (a recounted tile's block may not have started), so
// its blocks are counted instead: thread 0 of each block counts its block as
// started once it has used the epoch (a store of a value computed from it, or an
// LDS copy behind a barrier, has made the read complete; the count is relaxed: a
// release would write back the L2 of the XCD, about 1.5 us per block).  The block
// that finishes the last tile waits until all have started, then starts the next
// epoch.  A late block is one that waits for a slot, which frees as others finish.
__device__ __forceinline__ void mark_started(WsHeader* h)
{
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keeps the compiler from issuing it earlier
    __hip_atomic_fetch_add(&h->started, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void end_call(WsHeader* h, uint32_t epoch, uint32_t blocks)
{
    const uint64_t t0 = wall_clock64();
    // relaxed: the epoch store below is issued only after this loop has exited
    while (__hip_atomic_load(&h->started, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < blocks) {
        if (uint64_t(wall_clock64()) - t0 >= AWAIT_LIMIT_TICKS) {
            flag_error(h, WS_ERR_WAIT_TIMEOUT);
            break;
        }
        __builtin_amdgcn_s_sleep(8);
    }
    __hip_atomic_store(&h->started, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    start_next_epoch(h, epoch);
}

__device__ __forceinline__ void flag_error(WsHeader* h, uint32_t bits)
{
    __hip_atomic_fetch_or(&h->error_flags, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------- look-back
// Status codecs: how a 64-bit status word holds (flag, value) and how values of
// a window are combined across a wave.
//
// Scan values: the operator's 32-bit element in the low half.
template <class Op>
struct ScanCodec {
    using V = typename Op::T;
    static constexpr uint32_t EPOCH_MASK = (1u << 30) - 1u;
    static __device__ __forceinline__ uint32_t flag(uint64_t w, uint32_t ep)
    {
        return ((uint32_t(w >> 32) & EPOCH_MASK) == (ep & EPOCH_MASK)) ? uint32_t(w >> 62) : ST_EMPTY;
    }
    static __device__ __forceinline__ V value(uint64_t w) { return from_bits<V>(uint32_t(w)); }
    static __device__ __forceinline__ uint64_t pack(uint32_t f, V v, uint32_t ep)
    {
        return (uint64_t(f) << 62) | (uint64_t(ep & EPOCH_MASK) << 32) | uint64_t(to_bits(v));
    }
    static __device__ __forceinline__ V identity() { return Op::identity(); }
    static __device__ __forceinline__ V apply(V a, V b) { return Op::apply(a, b); }
    // whether a tile with this total publishes its full prefix itself
    static __device__ __forceinline__ bool self_published(V) { return false; }
    static __device__ __forceinline__ V wave_scan(V v) { return wave_inclusive_scan<Op>(v); }
    static __device__ __forceinline__ V lane(V v, int l) { return read_lane(v, l); }
    // Combine the lanes' partials in lane order (lanes below `hi` hold identity).
    static __device__ __forceinline__ V wave_reduce(V part, int /*hi*/)
    {
        return read_lane(wave_inclusive_scan<Op>(part), 63);
    }
};

// Compaction counts: a 36-bit count (n < 2^36 elements).  Tile totals are at
// most one tile's elements; only full prefixes are large.
// Word layout: flag 63..62, the count's bits 35..32 in 61..58, the epoch's low 26
// bits in 57..32, the count's bits 31..0 in 31..0.  Every codec keeps its epoch's
// low bits from bit 32 up, so that one workspace can serve scans, segmented scans
// and compactions in turn: a word that another codec wrote in an earlier call
// reads as empty unless the two epochs differ by a multiple of 2^26 (the count
// codec's epoch width).  (With the epoch above the whole 36-bit count, a count
// word written at epoch e read as epoch 16 e to the scan codec.)
struct CountCodec {
    using V = uint64_t;
    static constexpr uint64_t MASK = (uint64_t(1) << 36) - 1;
    static constexpr uint32_t EPOCH_MASK = (1u << 26) - 1u;
    static __device__ __forceinline__ uint32_t flag(uint64_t w, uint32_t ep)
    {
        return ((uint32_t(w >> 32) & EPOCH_MASK) == (ep & EPOCH_MASK)) ? uint32_t(w >> 62) : ST_EMPTY;
    }
    static __device__ __forceinline__ V value(uint64_t w)
    {
        return (((w >> 58) & 0xfull) << 32) | (w & 0xffffffffull);
    }
    static __device__ __forceinline__ uint64_t pack(uint32_t f, V v, uint32_t ep)
    {
        return (uint64_t(f) << 62) | (((v >> 32) & 0xfull) << 58) | (uint64_t(ep & EPOCH_MASK) << 32) |
               (v & 0xffffffffull);
    }
    static __device__ __forceinline__ V identity() { return 0; }
    static __device__ __forceinline__ V apply(V a, V b) { return a + b; }
    static __device__ __forceinline__ bool self_published(V) { return false; }
    // The chasing wave scans tile totals (each at most one tile, so 64 of them
    // fit in 32 bits) and adds the 64-bit base afterwards.
    static __device__ __forceinline__ V wave_scan(V v) { return wave_inclusive_scan<SumU32>(uint32_t(v)); }
    static __device__ __forceinline__ V lane(V v, int l)
    {
        const uint32_t lo = __builtin_amdgcn_readlane(uint32_t(v), l);
        const uint32_t hi = __builtin_amdgcn_readlane(uint32_t(v >> 32), l);
        return (uint64_t(hi) << 32) | lo;
    }
    // A lane's partial is small (a few tile counts) except on lane `hi`, whose
    // partial includes a full prefix; the small ones are summed in 32 bits, the
    // big one read whole.
    static __device__ __forceinline__ V wave_reduce(V part, int hi)
    {
        const uint32_t small = (lane_id() > hi) ? uint32_t(part) : 0u;
        V r = read_lane(wave_inclusive_scan<SumU32>(small), 63);
        if (hi >= 0)
            r += lane(part, hi);
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

// No fallback: a look-back that runs out of time gives up (tickets guarantee that
// this only happens on a defect) and reports it in the error word.
struct NoRecount {
};

// With a recount function (block-index tiles), a look-back that runs out of time
// computes the totals of the window's unpublished tiles itself (recount(j), called
// by the whole wave, must return tile j's exact total) and goes on.
template <class Codec, int WIDE = LB_WINDOW, class Recount = NoRecount>
__device__ typename Codec::V lookback(const uint64_t* status, int64_t tile, uint32_t ep, WsHeader* hdr,
                                      Recount recount = Recount())
{
    static_assert(WIDE >= LB_NEAR && WIDE <= LB_WINDOW, "a wide poll reads LB_NEAR to 64 tiles");
    using V = typename Codec::V;
    const int lane = lane_id();
    auto word = [&](int64_t idx) -> uint64_t {
        return idx >= 0 ? status_load(status + idx * STATUS_STRIDE) : Codec::pack(ST_PREFIX, Codec::identity(), ep);
    };
    if constexpr (WIDE > LB_NEAR) {
        // narrow first poll: lanes 56..63 read the eight nearest tiles; the
        // other lanes stand for tiles that do not take part (identity totals).
        // With WIDE == LB_NEAR the loop's first poll reads the same words.
        const bool near = lane >= LB_WINDOW - LB_NEAR;
        const uint64_t w = near ? word(tile - LB_WINDOW + lane) : Codec::pack(ST_AGGREGATE, Codec::identity(), ep);
        const uint64_t has = __ballot(near && Codec::flag(w, ep) == ST_PREFIX);
        const int hi = has ? 63 - __builtin_clzll(has) : -1;
        if (hi >= 0 && !__ballot(lane > hi && Codec::flag(w, ep) == ST_EMPTY))
            return Codec::wave_reduce(lane >= hi ? Codec::value(w) : Codec::identity(), hi);
    }
    V excl = Codec::identity();
    int64_t last = tile - 1;
    uint64_t t0 = wait_start();
    for (;;) {
        // lanes 64 - WIDE .. 63 read the WIDE newest tiles not yet combined
        const bool act = lane >= LB_WINDOW - WIDE;
        uint64_t w = act ? word(last - (LB_WINDOW - 1) + lane) : Codec::pack(ST_AGGREGATE, Codec::identity(), ep);
        const uint64_t has = __ballot(act && Codec::flag(w, ep) == ST_PREFIX);
        const int hi = has ? 63 - __builtin_clzll(has) : -1;
        uint64_t empty = __ballot(act && lane > hi && Codec::flag(w, ep) == ST_EMPTY);
        if (empty) {
            if (!wait_expired(t0, __is_same(Recount, NoRecount) ? WAIT_LIMIT_TICKS : FALLBACK_TICKS)) {
                __builtin_amdgcn_s_sleep(LB_SLEEP);
                continue;
            }
            if constexpr (__is_same(Recount, NoRecount)) {
                if (lane == 0)
                    flag_error(hdr, WS_ERR_WAIT_TIMEOUT);
                return excl;  // only reached on a defect; the error word reports it
            } else {
                while (empty) {  // the fallback: count the missing tiles here
                    const int m = __builtin_ctzll(empty);
                    empty &= empty - 1;
                    const typename Codec::V v = recount(last - (LB_WINDOW - 1) + m);
                    if (lane == m)
                        w = Codec::pack(ST_AGGREGATE, v, ep);
                }
            }
        }
        const V part = lane >= hi ? Codec::value(w) : Codec::identity();
        excl = Codec::apply(Codec::wave_reduce(part, hi), excl);  // older tiles on the left
        if (hi >= 0)
            return excl;
        last -= WIDE;
        t0 = wait_start();  // progress: the next window's wait starts afresh
    }
}

// ---------------------------------------------------------------- chased prefixes
// The single-pass scan does not let every tile walk back on its own.  One wave
// (the one that scanned tile 0) stays resident after its tile and moves the
// "full prefix" frontier forward for everyone: it polls the total words of the
// current group of 64 tiles, takes the run of consecutive tiles that have
// published their totals, scans them across the wave, and publishes a full prefix
// for each (chase_prefixes below).  Every other tile publishes its total and then
// polls one word, its predecessor's prefix word, until it holds the full prefix:
// its own exclusive prefix.  A tile slot holds two words: the prefix word (word
// 0, written only with full prefixes) and the total word (word TOTAL_WORD, the
// tile's own total, never overwritten).  Every writer of a word writes the same
// value, so the order of writes does not matter.  (Side by side in one cache line
// they measured 1 us faster on the 2^28 scan than on separate lines.)
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
// waiting for anything.  With tickets, a tile with an id is resident, so the
// frontier always reaches every tile; with block-index tiles a waiting tile that
// runs out of time replays the chaser's arithmetic itself (replay_prefix).
constexpr int TOTAL_WORD = 1;       // the total word's offset in a tile slot (64-bit words)
constexpr int LB_WAIT_SLEEP = 8;    // s_sleep units between a tile's polls of its predecessor
constexpr int LB_CHASE_SLEEP = 2;   // between chaser polls that found nothing new
constexpr int CHASE_GROUP = 64;     // tiles per group of the chaser's scans (one per lane)

__device__ __forceinline__ uint64_t* total_word(uint64_t* status, int64_t tile)
{
    return status + tile * STATUS_STRIDE + TOTAL_WORD;
}

// Waits for the full prefix of tile - 1 (tile >= 1): the exclusive prefix of
// `tile`.  Called by a whole wave; every lane reads the same word.  Returns false
// when the time limit passes first (`out` is then untouched).
template <class Codec>
__device__ bool wait_prefix(const uint64_t* status, int64_t tile, uint32_t ep, typename Codec::V& out,
                            uint64_t limit)
{
    const uint64_t* p = status + (tile - 1) * STATUS_STRIDE;
    const uint64_t t0 = wait_start();
    for (;;) {
        const uint64_t w = status_load(p);
        if (__ballot(Codec::flag(w, ep) == ST_PREFIX)) {
            out = Codec::value(w);
            return true;
        }
        if (wait_expired(t0, limit))
            return false;
        __builtin_amdgcn_s_sleep(LB_WAIT_SLEEP);
    }
}

// Publishes the full prefix of tiles 1 .. num_tiles - 1, in order, given the
// total of tile 0.  Called by one whole wave, after tile 0 is published.
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
// head) publishes it itself (Codec::self_published tells from its total); the
// wave's scan gives the same value there, and the wave does not write it again.
// A wait without progress past the time limit ends the wave silently: waiting
// tiles then run out of time themselves and either replay (block-index tiles) or
// report it (tickets).
// have0 = 1: lane 0 starts with tile 0's total (total0, the caller's own tile);
// have0 = 0: tile 0's total is polled like the others (total0 unused).
// AHEAD = 2: each poll also reads the next group's 64 total words (a second word
// per lane), so one poll can carry the frontier over up to 128 tiles.  The
// compaction needs it: its 16384-element tiles come at about 80 per microsecond,
// more than one group per poll round trip (about a microsecond) can follow.  The
// groups and their scans stay those of tile 0's alignment, so the values do not
// change with AHEAD.
template <class Codec, int AHEAD = 1>
__device__ void chase_prefixes(uint64_t* status, int64_t num_tiles, typename Codec::V total0, uint32_t ep,
                               int have0 = 1)
{
    static_assert(AHEAD == 1 || AHEAD == 2, "one or two groups per poll");
    using V = typename Codec::V;
    const int lane = lane_id();
    int64_t g0 = 0;                                  // first tile of the current group
    V base = Codec::identity();                      // full prefix of tile g0 - 1
    V tot[AHEAD];                                    // totals seen so far: group g0 (+ the next)
#pragma unroll
    for (int q = 0; q < AHEAD; ++q)
        tot[q] = Codec::identity();
    if (lane == 0 && have0)
        tot[0] = total0;
    int have = have0;                                // tiles g0 .. g0 + have - 1 hold their totals
    uint64_t t0 = wait_start();
    while (g0 + have < num_tiles) {
        uint64_t w[AHEAD];
        int k = 64 * AHEAD;                          // tiles g0 .. g0 + k - 1 now hold totals
#pragma unroll
        for (int q = 0; q < AHEAD; ++q) {
            const int pos = 64 * q + lane;
            const int64_t idx = g0 + pos;
            const bool want = pos >= have && idx < num_tiles;
            w[q] = want ? status_load(total_word(status, idx)) : 0ull;
            const bool ready = pos < have || (want && Codec::flag(w[q], ep) == ST_AGGREGATE);
            const uint64_t miss = __ballot(!ready);
            if (miss && k == 64 * AHEAD)
                k = 64 * q + __builtin_ctzll(miss);
        }
        if (k == have) {
            if (wait_expired(t0))
                return;
            __builtin_amdgcn_s_sleep(LB_CHASE_SLEEP);
            continue;
        }
        t0 = wait_start();
        V b = base;
#pragma unroll
        for (int q = 0; q < AHEAD; ++q) {
            const int pos = 64 * q + lane;
            if (pos >= have && pos < k)
                tot[q] = Codec::value(w[q]);
            if (64 * q < k) {
                // older on the left: b (+) totals of the group's tiles up to this lane
                const int kq = k - 64 * q < 64 ? k - 64 * q : 64;
                const V inc = Codec::apply(b, Codec::wave_scan(lane < kq ? tot[q] : Codec::identity()));
                if (pos >= have && pos < k && !Codec::self_published(tot[q]))
                    status_store(status + (g0 + pos) * STATUS_STRIDE, Codec::pack(ST_PREFIX, inc, ep));
                if (kq == 64)
                    b = Codec::lane(inc, 63);
            }
        }
        have = k;
        while (have >= 64) {  // group g0 complete: slide by one group
            base = Codec::lane(Codec::apply(base, Codec::wave_scan(tot[0])), 63);
            g0 += 64;
            have -= 64;
#pragma unroll
            for (int q = 0; q + 1 < AHEAD; ++q)
                tot[q] = tot[q + 1];
            tot[AHEAD - 1] = Codec::identity();
        }
    }
}

// The full prefix of tile `last` exactly as chase_prefixes computes it, by one
// wave that depends on no other block: the fallback of a block-index tile whose
// wait ran out of time.  Group bases come from published prefix words where they
// exist (a group's base is the full prefix of the tile before it); tile totals
// from total words, or, for a tile that has not published one, from
// total_of(j), which must compute the total exactly as tile j's own block does
// (the same operations in the same order, so float results match bit for bit).
// The full prefixes it computes (each group end it passes, and `last`) are
// published on the way: the same values the chasing wave writes.  Totals are not:
// a total word is only ever written by its tile's own block, so a published total
// also says that block has started (read the call's epoch).
template <class Codec, class TotalFn>
__device__ typename Codec::V replay_prefix(uint64_t* status, int64_t last, uint32_t ep, TotalFn total_of)
{
    using V = typename Codec::V;
    const int lane = lane_id();
    const int64_t g = last / CHASE_GROUP;
    // the latest group at or before g whose base is published (group 0's is the identity)
    int64_t gb = g;
    V base = Codec::identity();
    for (; gb > 0; --gb) {
        const uint64_t w = status_load(status + (gb * CHASE_GROUP - 1) * STATUS_STRIDE);
        if (Codec::flag(w, ep) == ST_PREFIX) {
            base = Codec::value(w);
            break;
        }
    }
    for (int64_t gg = gb;; ++gg) {
        const int64_t first = gg * CHASE_GROUP;
        const int64_t idx = first + lane;
        const bool want = idx <= last;
        const uint64_t w = want ? status_load(total_word(status, idx)) : 0ull;
        V tot = want && Codec::flag(w, ep) == ST_AGGREGATE ? Codec::value(w) : Codec::identity();
        uint64_t missing = __ballot(want && Codec::flag(w, ep) != ST_AGGREGATE);
        while (missing) {
            const int m = __builtin_ctzll(missing);
            missing &= missing - 1;
            const V v = total_of(first + m);  // the whole wave computes it
            if (lane == m)
                tot = v;
        }
        const V inc = Codec::apply(base, Codec::wave_scan(tot));
        if (gg == g) {
            const int l = int(last - first);
            if (lane == l)
                status_store(status + idx * STATUS_STRIDE, Codec::pack(ST_PREFIX, inc, ep));
            return Codec::lane(inc, l);
        }
        base = Codec::lane(inc, CHASE_GROUP - 1);
        if (lane == CHASE_GROUP - 1)
            status_store(status + idx * STATUS_STRIDE, Codec::pack(ST_PREFIX, inc, ep));
    }
}

// Waits until tiles 0 .. last-1 have each published their own total under epoch
// `ep` (see the block-index tiles above).  One whole wave.
template <class Codec>
__device__ void await_totals(uint64_t* status, int64_t last, uint32_t ep, WsHeader* hdr)
{
    const uint64_t t0 = wall_clock64();
    for (int64_t first = 0; first < last; first += 64) {
        const int64_t idx = first + lane_id();
        for (;;) {
            const bool ok = idx >= last || Codec::flag(status_load(total_word(status, idx)), ep) == ST_AGGREGATE;
            if (!__ballot(!ok))
                break;
            if (uint64_t(wall_clock64()) - t0 >= AWAIT_LIMIT_TICKS) {
                if (lane_id() == 0)
                    flag_error(hdr, WS_ERR_WAIT_TIMEOUT);
                return;
            }
            __builtin_amdgcn_s_sleep(8);
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
__device__ typename Codec::V lookback_grouped(const uint64_t* status, int64_t tile, uint32_t ep, WsHeader* hdr)
{
    const int lane = lane_id();
    const int64_t g0 = tile - tile % LB_GROUP;  // first tile of this tile's group
    const int before = int(tile - g0);         // tiles of the group before this one
    const bool needed = lane == 0 ? g0 > 0 : lane <= before;
    const int64_t idx = lane == 0 ? g0 - 1 : g0 + lane - 1;
    const uint64_t t0 = wait_start();
    for (;;) {
        const uint64_t w = needed ? status_load(status + idx * STATUS_STRIDE)
                                  : Codec::pack(ST_AGGREGATE, Codec::identity(), ep);
        const uint32_t f = Codec::flag(w, ep);
        const bool ready = !needed || (lane == 0 ? f == ST_PREFIX : f != ST_EMPTY);
        if (!__ballot(!ready))
            return Codec::wave_reduce(needed ? Codec::value(w) : Codec::identity(), -1);
        if (wait_expired(t0)) {
            if (lane == 0)
                flag_error(hdr, WS_ERR_WAIT_TIMEOUT);
            return Codec::identity();  // only reached on a defect; the error word reports it
        }
        __builtin_amdgcn_s_sleep(LB_SLEEP);
    }
}

}  // namespace ls
