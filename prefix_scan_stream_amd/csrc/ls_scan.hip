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
//   3. its first wave looks back over the 64 preceding tiles at a time, summing
//      published totals until it meets a tile that has published its full
//      prefix, then publishes its own full prefix;
//   4. it writes prefix (+) local scan with 128-bit stores.
// Each tile status is one 64-bit word (flag + value) so a single atomic access
// carries both; see ls_device.hpp.
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

constexpr int SCAN_BLOCK = 256;                       // 4 waves
constexpr int SCAN_WAVES = SCAN_BLOCK / 64;
constexpr int SCAN_CHUNKS = 4;                        // 128-bit runs per thread
constexpr int SCAN_TILE = SCAN_BLOCK * SCAN_CHUNKS * 4;  // 4096 elements

static_assert(SCAN_WAVES * SCAN_CHUNKS <= 64, "run totals must fit one wave");

template <class T>
__device__ __forceinline__ uint64_t pack32(uint32_t flag, T v)
{
    return (uint64_t(flag) << 32) | uint64_t(to_bits(v));
}

// Exclusive prefix of tile `tile` (>= 1) from the tile status words.  Runs on one
// full wave.  Window: lanes 0..63 look at tiles last-63 .. last.  If some lane sees
// a full prefix, the highest such lane ends the walk: the answer is the operator
// over that lane and all lanes above it.  Otherwise all 64 totals are combined and
// the window moves 64 tiles back.  Any empty word at or above the stopping lane
// means a predecessor has not published yet: poll again.
template <class Op>
__device__ typename Op::T lookback_prefix(const uint64_t* status, int64_t tile, WsHeader* hdr)
{
    using T = typename Op::T;
    const int lane = lane_id();
    T excl = Op::identity();
    int64_t last = tile - 1;
    int spins = 0;
    for (;;) {
        const int64_t idx = last - 63 + lane;
        const uint64_t w = (idx >= 0) ? status_load(status + idx) : pack32(ST_PREFIX, Op::identity());
        const uint32_t flag = uint32_t(w >> 32);
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
            return excl;  // only reached on a defect; the error word reports it
        }
        const T v = (lane >= hi) ? from_bits<T>(uint32_t(w)) : Op::identity();
        const T r = read_lane(wave_inclusive_scan<Op>(v), 63);
        excl = Op::apply(r, excl);  // older tiles on the left
        if (hi >= 0)
            return excl;
        last -= 64;
    }
}

template <class Op, bool INCLUSIVE, bool VEC>
__global__ __launch_bounds__(SCAN_BLOCK) void scan_single_pass_kernel(
    const typename Op::T* in, typename Op::T* out, int64_t n, int64_t num_tiles, WsHeader* hdr,
    uint64_t* status, typename Op::T* total)
{
    using T = typename Op::T;
    __shared__ T s_tot[SCAN_CHUNKS][SCAN_WAVES];
    __shared__ uint32_t s_tile;
    __shared__ T s_prefix;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const T id = Op::identity();

    if (tid == 0)
        s_tile = take_tile_id(hdr);
    __syncthreads();
    const int64_t tile = s_tile;
    const int64_t tbase = tile * SCAN_TILE;

    // 1. load: run j of thread t covers elements tbase + 4*(j*BLOCK + t) + 0..3
    Run4<T> r[SCAN_CHUNKS];
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j)
        r[j] = load_run<T, VEC>(in, tbase + 4 * int64_t(j * SCAN_BLOCK + tid), n, id);

    // 2. serial inclusive scan of each run, then a wave scan of the run totals
    T wex[SCAN_CHUNKS];
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j) {
        r[j].v[1] = Op::apply(r[j].v[0], r[j].v[1]);
        r[j].v[2] = Op::apply(r[j].v[1], r[j].v[2]);
        r[j].v[3] = Op::apply(r[j].v[2], r[j].v[3]);
        const T inc = wave_inclusive_scan<Op>(r[j].v[3]);
        wex[j] = wave_shift_up<Op>(inc);
        if (lane == 63)
            s_tot[j][wave] = inc;
    }
    __syncthreads();

    // the (run, wave) totals in element order: run-major, then wave
    T pre[SCAN_CHUNKS];
    T agg = id;
#pragma unroll
    for (int jj = 0; jj < SCAN_CHUNKS; ++jj) {
#pragma unroll
        for (int ww = 0; ww < SCAN_WAVES; ++ww) {
            if (ww == wave)
                pre[jj] = agg;
            agg = Op::apply(agg, s_tot[jj][ww]);
        }
    }

    // 3. publish and look back
    if (wave == 0) {
        T p = id;
        if (tile == 0) {
            if (lane == 0)
                status_store(status, pack32(ST_PREFIX, agg));
        } else {
            if (lane == 0)
                status_store(status + tile, pack32(ST_AGGREGATE, agg));
            p = lookback_prefix<Op>(status, tile, hdr);
            if (lane == 0)
                status_store(status + tile, pack32(ST_PREFIX, Op::apply(p, agg)));
        }
        if (lane == 0)
            s_prefix = p;
    }
    __syncthreads();
    const T tp = s_prefix;

    // 4. finish and store
#pragma unroll
    for (int j = 0; j < SCAN_CHUNKS; ++j) {
        const T cp = Op::apply(tp, Op::apply(pre[j], wex[j]));
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
        store_run<T, VEC>(out, tbase + 4 * int64_t(j * SCAN_BLOCK + tid), n, o);
    }
    if (total != nullptr && tile == num_tiles - 1 && tid == 0)
        *total = Op::apply(tp, agg);
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
