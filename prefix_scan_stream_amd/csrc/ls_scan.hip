// ls_scan.hip -- single-pass device-wide scan with decoupled look-back (gfx950).
//
// The parallel prefix scan page (geek-doc.cn, section 四) composes a large scan
// from per-block scans, a scan of the block totals, and a pass that adds each
// block's offset -- three launches, with the whole array read twice and written
// twice.  The same page mentions, and sets aside, letting blocks hand their
// totals to one another inside one launch through flags in global memory.  That
// is the design used here, because only it moves the minimum 2*n*4 bytes that
// bound an HBM-limited scan:
//   1. a block takes the next tile id (start order, so it only ever waits for
//      blocks already running) and loads its tile with 128-bit loads;
//   2. it scans the tile in registers (serial runs of 4, DPP wave scan, LDS scan
//      of the per-wave totals) and publishes the tile total;
//   3. its first wave looks back over the preceding tiles, 256 per poll,
//      combining published totals until it meets a tile that has published its
//      full prefix, then publishes its own full prefix;
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
constexpr int SCAN_TILE = SCAN_BLOCK * SCAN_CHUNKS * 4;  // 16384 elements by default

static_assert(SCAN_WAVES * SCAN_CHUNKS <= 64, "the (run, wave) totals are scanned by one wave");

// Tile-local part of the scan, shared by every tile a block processes: serial
// scan of each run, wave scan of the run totals (exclusive result in wex), and
// the (run, wave) totals left in LDS by lane 63, in element order.
template <class Op>
__device__ __forceinline__ void scan_tile_local(Run4<typename Op::T> (&r)[SCAN_CHUNKS],
                                                typename Op::T (&wex)[SCAN_CHUNKS],
                                                typename Op::T* s_part, int lane, int wave)
{
    using T = typename Op::T;
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j) {
        r[j].v[1] = Op::apply(r[j].v[0], r[j].v[1]);
        r[j].v[2] = Op::apply(r[j].v[1], r[j].v[2]);
        r[j].v[3] = Op::apply(r[j].v[2], r[j].v[3]);
        const T inc = wave_inclusive_scan<Op>(r[j].v[3]);
        wex[j] = wave_shift_up<Op>(inc);
        if (lane == 63)
            s_part[j * SCAN_WAVES + wave] = inc;
    }
}

#ifndef LS_SCAN_LDS_RESERVE
#define LS_SCAN_LDS_RESERVE 0
#endif

// One tile per block; blocks take tile ids in the order they start.
template <class Op, bool INCLUSIVE, bool VEC>
__global__ __launch_bounds__(SCAN_BLOCK) void scan_single_pass_kernel(
    const typename Op::T* in, typename Op::T* out, int64_t n, int64_t num_tiles, WsHeader* hdr,
    uint64_t* status, typename Op::T* total)
{
    using T = typename Op::T;
    using Codec = ScanCodec<Op>;
    constexpr int PARTS = SCAN_CHUNKS * SCAN_WAVES;  // (run, wave) partial totals per tile
    constexpr uint32_t RUN_STRIDE = SCAN_BLOCK * 16u;
    __shared__ T s_part[PARTS + LS_SCAN_LDS_RESERVE];
    __shared__ uint32_t s_tile;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const T id = Op::identity();

    if (tid == 0)
        s_tile = take_tile_id(hdr);
    __syncthreads();
    const int64_t tile = s_tile;
    const int64_t tbase = tile * SCAN_TILE;
    const int64_t rem = n - tbase;
    const uint32_t valid = rem < SCAN_TILE ? uint32_t(rem) : uint32_t(SCAN_TILE);
    const bool full = valid == SCAN_TILE;
    const __amdgpu_buffer_rsrc_t rin = make_rsrc(in + tbase, valid * 4u);
    const __amdgpu_buffer_rsrc_t rout = make_rsrc(out + tbase, valid * 4u);
    const uint32_t voff = uint32_t(tid) * 16u;  // run j of thread t: elements 4*(j*BLOCK + t) + 0..3

    // 1. load.  Elements past n (last tile only) read as 0; they sit after every
    // valid element in scan order, so no output below n depends on them.  The
    // four element loads of a run are merged into one 128-bit access.
    Run4<T> r[SCAN_CHUNKS];
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j)
        r[j] = load_run_x1<T>(rin, voff, j * RUN_STRIDE);

    // 2. local scan: runs, wave scan of run totals, (run, wave) totals to LDS
    T wex[SCAN_CHUNKS];
    scan_tile_local<Op>(r, wex, s_part, lane, wave);
    __syncthreads();

    // 3. wave 0: scan the partial totals (one per lane), publish the tile total,
    // look back for the tile prefix, and leave prefix (+) partial-exclusive in LDS.
    if (wave == 0) {
        const T v = lane < PARTS ? s_part[lane] : id;
        const T inc = wave_inclusive_scan<Op>(v);
        const T exc = wave_shift_up<Op>(inc);
        const T agg = read_lane(inc, 63);
        T p = id;
        if (tile == 0) {
            if (lane == 0)
                status_store(status, Codec::pack(ST_PREFIX, agg));
        } else {
            if (lane == 0)
                status_store(status + tile, Codec::pack(ST_AGGREGATE, agg));
            p = lookback<Codec>(status, tile, hdr);
            if (lane == 0)
                status_store(status + tile, Codec::pack(ST_PREFIX, Op::apply(p, agg)));
        }
        if (lane < PARTS)
            s_part[lane] = Op::apply(p, exc);
    }
    __syncthreads();

    // 4. finish and store; the thread holding element n-1 writes the total
    const int64_t last_local = (tile == num_tiles - 1) ? int64_t(valid) - 1 : -1;
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
        if (total != nullptr) {
            // select, not index: a run-time index into r[] would move the whole
            // tile from registers to per-lane scratch memory
            const int64_t kk = last_local - 4 * int64_t(j * SCAN_BLOCK + tid);
            if (kk >= 0 && kk < 4) {
                T v = r[j].v[0];
#pragma unroll
                for (int k = 1; k < 4; ++k)
                    v = (kk == k) ? r[j].v[k] : v;
                *total = Op::apply(cp, v);
            }
        }
    }
}

// Clears the workspace header and the first `words` status words.
__global__ __launch_bounds__(256) void ws_clear_kernel(uint4* p, int64_t n16)
{
    const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (i < n16)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

__global__ void store_u32_kernel(uint32_t* p, uint32_t v)
{
    if (threadIdx.x == 0 && blockIdx.x == 0)
        *p = v;
}

// ------------------------------------------------------------------ host side

int64_t scan_tile_elems() { return SCAN_TILE; }

static int64_t num_tiles_for(int64_t n) { return (n + SCAN_TILE - 1) / SCAN_TILE; }

size_t scan_workspace_bytes(int64_t n)
{
    int64_t tiles = num_tiles_for(n);
    if (tiles < 1)
        tiles = 1;
    size_t bytes = sizeof(WsHeader) + size_t(tiles) * sizeof(uint64_t);
    return (bytes + 255) & ~size_t(255);
}

hipError_t clear_workspace(void* ws, int64_t status_words, hipStream_t s)
{
    const int64_t bytes = int64_t(sizeof(WsHeader)) + status_words * 8;
    const int64_t n16 = (bytes + 15) / 16;
    const int64_t blocks = (n16 + 255) / 256;
    hipLaunchKernelGGL(ws_clear_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                       reinterpret_cast<uint4*>(ws), n16);
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

template <class Op>
static hipError_t run_scan(const void* in, void* out, int64_t n, bool inclusive, void* total,
                           void* ws, hipStream_t s)
{
    using T = typename Op::T;
    if (n == 0) {
        if (total)
            hipLaunchKernelGGL(store_u32_kernel, dim3(1), dim3(64), 0, s,
                               reinterpret_cast<uint32_t*>(total), identity_bits<Op>());
        return hipGetLastError();
    }
    const int64_t tiles = num_tiles_for(n);
    hipError_t e = clear_workspace(ws, tiles, s);
    if (e != hipSuccess)
        return e;
    auto* hdr = reinterpret_cast<WsHeader*>(ws);
    auto* status = reinterpret_cast<uint64_t*>(reinterpret_cast<char*>(ws) + sizeof(WsHeader));
    const bool vec = ((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0;
    const T* pin = reinterpret_cast<const T*>(in);
    T* pout = reinterpret_cast<T*>(out);
    T* ptot = reinterpret_cast<T*>(total);
    const dim3 grid(static_cast<uint32_t>(tiles)), block(SCAN_BLOCK);
    if (inclusive) {
        if (vec)
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, true, true>), grid, block, 0, s, pin, pout,
                               n, tiles, hdr, status, ptot);
        else
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, true, false>), grid, block, 0, s, pin,
                               pout, n, tiles, hdr, status, ptot);
    } else {
        if (vec)
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, false, true>), grid, block, 0, s, pin,
                               pout, n, tiles, hdr, status, ptot);
        else
            hipLaunchKernelGGL((scan_single_pass_kernel<Op, false, false>), grid, block, 0, s, pin,
                               pout, n, tiles, hdr, status, ptot);
    }
    return hipGetLastError();
}

hipError_t launch_scan(const void* in, void* out, int64_t n, int dtype, int op, bool inclusive,
                       void* total, void* ws, hipStream_t s)
{
    switch (op) {
    case OP_SUM:
        if (dtype == DT_FLOAT32)
            return run_scan<SumF32>(in, out, n, inclusive, total, ws, s);
        return run_scan<SumU32>(in, out, n, inclusive, total, ws, s);
    case OP_XOR:
        return run_scan<XorU32>(in, out, n, inclusive, total, ws, s);
    case OP_MAX:
        if (dtype == DT_INT32)
            return run_scan<MaxI32>(in, out, n, inclusive, total, ws, s);
        if (dtype == DT_UINT32)
            return run_scan<MaxU32>(in, out, n, inclusive, total, ws, s);
        return run_scan<MaxF32>(in, out, n, inclusive, total, ws, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ls
