// ls_batched.hip -- row-wise scan of a row-major matrix, no carry between rows.
//
// The uniform-length case of a segmented scan (lpnh.cn parallel scan overview,
// section 7.2).  Rows are independent, so there is no inter-block communication
// at all; the two shapes follow the page hierarchy of the parallel prefix scan
// page (geek-doc.cn, section 五: a warp-level scan for short rows, a warp scan
// plus a scan of the per-warp totals for block-sized rows):
//   - cols <= 64: one row per 16-lane DPP row.  Each lane holds 4 consecutive
//     elements (one 128-bit word when aligned), scans them serially, and a
//     4-step row_shr scan combines the 16 lanes.  A wave covers 4 rows per pass;
//     each thread makes ROW16_PASSES passes, loads first, to keep many 128-bit
//     loads in flight.  Float32 additions per output: at most 3 + 4 + 1.
//   - cols > 64: one block per row, in chunks of 1024 elements (256 threads x 4)
//     with a running carry across chunks.  The block-level step has four
//     interchangeable forms (BlockScanKind below), selected by the caller.
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

constexpr int ROW16_BLOCK = 256;
constexpr int ROW16_PASSES = 4;
constexpr int ROW16_ROWS_PER_BLOCK = (ROW16_BLOCK / 16) * ROW16_PASSES;  // 64

template <class Op, bool EXCL, bool VEC>
__global__ __launch_bounds__(ROW16_BLOCK) void batched_row16_kernel(const typename Op::T* in,
                                                                    typename Op::T* out,
                                                                    int64_t rows, int cols)
{
    using T = typename Op::T;
    const T id = Op::identity();
    const int sub = threadIdx.x & 15;       // lane inside the 16-lane row
    const int grp = threadIdx.x >> 4;       // which of the block's 16 row slots
    const int64_t row0 = int64_t(blockIdx.x) * ROW16_ROWS_PER_BLOCK;
    const int c0 = sub * 4;

    Run4<T> r[ROW16_PASSES];
#pragma unroll
    for (int p = 0; p < ROW16_PASSES; ++p) {
        const int64_t row = row0 + p * (ROW16_BLOCK / 16) + grp;
        if (row < rows) {
            r[p] = load_run<T, VEC>(in + row * cols, c0, cols, id);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                r[p].v[k] = id;
        }
    }
#pragma unroll
    for (int p = 0; p < ROW16_PASSES; ++p) {
        r[p].v[1] = Op::apply(r[p].v[0], r[p].v[1]);
        r[p].v[2] = Op::apply(r[p].v[1], r[p].v[2]);
        r[p].v[3] = Op::apply(r[p].v[2], r[p].v[3]);
        const T inc = row16_inclusive_scan<Op>(r[p].v[3]);
        const T lex = row16_shift_up<Op>(inc);
        Run4<T> o;
        if constexpr (EXCL) {
            o.v[0] = lex;
#pragma unroll
            for (int k = 1; k < 4; ++k)
                o.v[k] = Op::apply(lex, r[p].v[k - 1]);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o.v[k] = Op::apply(lex, r[p].v[k]);
        }
        const int64_t row = row0 + p * (ROW16_BLOCK / 16) + grp;
        if (row < rows)
            store_run<T, VEC>(out + row * cols, c0, cols, o);
    }
}

constexpr int ROWB_BLOCK = 256;
constexpr int ROWB_WAVES = ROWB_BLOCK / 64;
constexpr int ROWB_CHUNK = ROWB_BLOCK * 4;

// ---- block-level scans of one value per thread (the thread's run total) ------
// Each returns the exclusive prefix of `v` over the block's threads, in thread
// order, and sets `total` to the block's reduction.  All threads must call it.
// The structs hold only LDS storage; `par` is per-thread state of the caller.
// Four ways, measured against each other on block-sized rows:
//   BS_WAVE_DPP    DPP scan inside each wave, wave totals through LDS: 1 barrier
//                  (the two-level shuffle scan of geek-doc.cn section 五);
//   BS_HS          Hillis-Steele over LDS, read / barrier / write / barrier per
//                  step: 2 x 8 barriers (geek-doc.cn section 二);
//   BS_HS_DOUBLE   Hillis-Steele with two LDS buffers, one barrier per step
//                  (same section, the double-buffer form);
//   BS_BLELLOCH    up-sweep, cleared root, down-sweep over LDS, 2 x 8 + 1
//                  barriers (geek-doc.cn section 三; pgsm.cn section 5.4).  The
//                  pair indices ai = offset (2 tid + 1) - 1, bi = offset (2 tid + 2) - 1
//                  at each level follow the pseudo-code of the lpnh.cn parallel scan
//                  overview, section 2.3; here every index is padded by one word per
//                  32, which leaves each level's active lanes on distinct LDS banks
//                  (rocprofv3 SQ_LDS_BANK_CONFLICT reads 0 for all four variants).
enum BlockScanKind : int { BS_WAVE_DPP = 0, BS_HS = 1, BS_HS_DOUBLE = 2, BS_BLELLOCH = 3 };

template <class Op, int KIND>
struct BlockScan;

template <class Op>
struct BlockScan<Op, BS_WAVE_DPP> {
    using T = typename Op::T;
    T s_tot[2][ROWB_WAVES];
    __device__ T exclusive(T v, T& total, int& par)
    {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const T inc = wave_inclusive_scan<Op>(v);
        const T wex = wave_shift_up<Op>(inc);
        if (lane == 63)
            s_tot[par][wave] = inc;
        __syncthreads();
        T pre = Op::identity(), agg = Op::identity();
#pragma unroll
        for (int ww = 0; ww < ROWB_WAVES; ++ww) {
            if (ww == wave)
                pre = agg;
            agg = Op::apply(agg, s_tot[par][ww]);
        }
        par ^= 1;  // the next call writes the other half: no second barrier needed
        total = agg;
        return Op::apply(pre, wex);
    }
};

template <class Op>
struct BlockScan<Op, BS_HS> {
    using T = typename Op::T;
    T s[ROWB_BLOCK];
    __device__ T exclusive(T v, T& total, int&)
    {
        const int tid = threadIdx.x;
        s[tid] = v;
        __syncthreads();
#pragma unroll
        for (int k = 1; k < ROWB_BLOCK; k <<= 1) {
            const T mine = s[tid];
            const T left = tid >= k ? s[tid - k] : Op::identity();
            __syncthreads();  // everyone has read the old values
            s[tid] = Op::apply(left, mine);
            __syncthreads();  // everyone has written the new ones
        }
        const T ex = tid > 0 ? s[tid - 1] : Op::identity();
        total = s[ROWB_BLOCK - 1];
        __syncthreads();  // s is rewritten by the next call
        return ex;
    }
};

template <class Op>
struct BlockScan<Op, BS_HS_DOUBLE> {
    using T = typename Op::T;
    T s[2][ROWB_BLOCK];
    __device__ T exclusive(T v, T& total, int&)
    {
        const int tid = threadIdx.x;
        int src = 0;
        s[0][tid] = v;
        __syncthreads();
#pragma unroll
        for (int k = 1; k < ROWB_BLOCK; k <<= 1) {
            const T mine = s[src][tid];
            s[src ^ 1][tid] = tid >= k ? Op::apply(s[src][tid - k], mine) : mine;
            src ^= 1;
            __syncthreads();
        }
        const T ex = tid > 0 ? s[src][tid - 1] : Op::identity();
        total = s[src][ROWB_BLOCK - 1];
        __syncthreads();
        return ex;
    }
};

template <class Op>
struct BlockScan<Op, BS_BLELLOCH> {
    using T = typename Op::T;
    static constexpr int PAD_SHIFT = 5;  // one pad word per 32 words
    T s[ROWB_BLOCK + (ROWB_BLOCK >> PAD_SHIFT)];
    static __device__ __forceinline__ int at(int i) { return i + (i >> PAD_SHIFT); }
    __device__ T exclusive(T v, T& total, int&)
    {
        const int tid = threadIdx.x;
        s[at(tid)] = v;
        __syncthreads();
        // up-sweep: each level folds the left half of a pair into the right half
        int offset = 1;
#pragma unroll
        for (int d = ROWB_BLOCK >> 1; d > 0; d >>= 1) {
            if (tid < d) {
                const int ai = offset * (2 * tid + 1) - 1;
                const int bi = offset * (2 * tid + 2) - 1;
                s[at(bi)] = Op::apply(s[at(ai)], s[at(bi)]);
            }
            offset <<= 1;
            __syncthreads();
        }
        total = s[at(ROWB_BLOCK - 1)];
        __syncthreads();
        if (tid == 0)
            s[at(ROWB_BLOCK - 1)] = Op::identity();  // cleared root: the scan is exclusive
        __syncthreads();
        // down-sweep: left child takes the parent's value, right child takes
        // parent (+) the left child's old total
#pragma unroll
        for (int d = 1; d < ROWB_BLOCK; d <<= 1) {
            offset >>= 1;
            if (tid < d) {
                const int ai = offset * (2 * tid + 1) - 1;
                const int bi = offset * (2 * tid + 2) - 1;
                const T left = s[at(ai)];
                s[at(ai)] = s[at(bi)];
                s[at(bi)] = Op::apply(s[at(bi)], left);
            }
            __syncthreads();
        }
        const T ex = s[at(tid)];
        __syncthreads();
        return ex;
    }
};

template <class Op, bool EXCL, bool VEC, int KIND>
__global__ __launch_bounds__(ROWB_BLOCK) void batched_block_kernel(const typename Op::T* in,
                                                                   typename Op::T* out, int64_t rows,
                                                                   int64_t cols)
{
    using T = typename Op::T;
    __shared__ BlockScan<Op, KIND> bs;
    const T id = Op::identity();
    const int tid = threadIdx.x;
    int par = 0;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const T* rin = in + row * cols;
        T* rout = out + row * cols;
        T carry = id;
        for (int64_t c0 = 0; c0 < cols; c0 += ROWB_CHUNK) {
            const int64_t idx = c0 + 4 * int64_t(tid);
            Run4<T> r = load_run<T, VEC>(rin, idx, cols, id);
            r.v[1] = Op::apply(r.v[0], r.v[1]);
            r.v[2] = Op::apply(r.v[1], r.v[2]);
            r.v[3] = Op::apply(r.v[2], r.v[3]);
            T agg;
            const T pre = bs.exclusive(r.v[3], agg, par);
            const T cp = Op::apply(carry, pre);
            Run4<T> o;
            if constexpr (EXCL) {
                o.v[0] = cp;
#pragma unroll
                for (int k = 1; k < 4; ++k)
                    o.v[k] = Op::apply(cp, r.v[k - 1]);
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    o.v[k] = Op::apply(cp, r.v[k]);
            }
            store_run<T, VEC>(rout, idx, cols, o);
            carry = Op::apply(carry, agg);
        }
    }
}

// ------------------------------------------------------------------ host side

template <class Op, bool EXCL, bool VEC>
static void launch_block_variant(const typename Op::T* pin, typename Op::T* pout, int64_t rows,
                                 int64_t cols, int kind, dim3 grid, hipStream_t s)
{
    const dim3 block(ROWB_BLOCK);
    switch (kind) {
    case BS_HS:
        hipLaunchKernelGGL((batched_block_kernel<Op, EXCL, VEC, BS_HS>), grid, block, 0, s, pin, pout, rows, cols);
        break;
    case BS_HS_DOUBLE:
        hipLaunchKernelGGL((batched_block_kernel<Op, EXCL, VEC, BS_HS_DOUBLE>), grid, block, 0, s, pin, pout, rows, cols);
        break;
    case BS_BLELLOCH:
        hipLaunchKernelGGL((batched_block_kernel<Op, EXCL, VEC, BS_BLELLOCH>), grid, block, 0, s, pin, pout, rows, cols);
        break;
    default:
        hipLaunchKernelGGL((batched_block_kernel<Op, EXCL, VEC, BS_WAVE_DPP>), grid, block, 0, s, pin, pout, rows, cols);
        break;
    }
}

template <class Op>
static hipError_t run_batched(const void* in, void* out, int64_t rows, int64_t cols, bool excl,
                              int kind, hipStream_t s)
{
    using T = typename Op::T;
    const T* pin = reinterpret_cast<const T*>(in);
    T* pout = reinterpret_cast<T*>(out);
    const bool vec = (((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0) &&
                     (cols % 4 == 0);
    if (cols <= 64 && kind == BS_WAVE_DPP) {
        const int64_t blocks = (rows + ROW16_ROWS_PER_BLOCK - 1) / ROW16_ROWS_PER_BLOCK;
        const dim3 grid(static_cast<uint32_t>(blocks)), block(ROW16_BLOCK);
        const int c = int(cols);
        if (excl) {
            if (vec)
                hipLaunchKernelGGL((batched_row16_kernel<Op, true, true>), grid, block, 0, s, pin, pout, rows, c);
            else
                hipLaunchKernelGGL((batched_row16_kernel<Op, true, false>), grid, block, 0, s, pin, pout, rows, c);
        } else {
            if (vec)
                hipLaunchKernelGGL((batched_row16_kernel<Op, false, true>), grid, block, 0, s, pin, pout, rows, c);
            else
                hipLaunchKernelGGL((batched_row16_kernel<Op, false, false>), grid, block, 0, s, pin, pout, rows, c);
        }
        return hipGetLastError();
    }
    const int64_t max_grid = int64_t(1) << 30;
    const dim3 grid(static_cast<uint32_t>(rows < max_grid ? rows : max_grid));
    if (excl) {
        if (vec)
            launch_block_variant<Op, true, true>(pin, pout, rows, cols, kind, grid, s);
        else
            launch_block_variant<Op, true, false>(pin, pout, rows, cols, kind, grid, s);
    } else {
        if (vec)
            launch_block_variant<Op, false, true>(pin, pout, rows, cols, kind, grid, s);
        else
            launch_block_variant<Op, false, false>(pin, pout, rows, cols, kind, grid, s);
    }
    return hipGetLastError();
}

hipError_t launch_batched(const void* in, void* out, int64_t rows, int64_t cols, int dtype, int op,
                          bool excl, int kind, hipStream_t s)
{
    if (rows == 0 || cols == 0)
        return hipSuccess;
    switch (op) {
    case OP_SUM:
        if (dtype == DT_FLOAT32)
            return run_batched<SumF32>(in, out, rows, cols, excl, kind, s);
        return run_batched<SumU32>(in, out, rows, cols, excl, kind, s);
    case OP_XOR:
        return run_batched<XorU32>(in, out, rows, cols, excl, kind, s);
    case OP_MAX:
        if (dtype == DT_INT32)
            return run_batched<MaxI32>(in, out, rows, cols, excl, kind, s);
        if (dtype == DT_UINT32)
            return run_batched<MaxU32>(in, out, rows, cols, excl, kind, s);
        return run_batched<MaxF32>(in, out, rows, cols, excl, kind, s);
    case OP_MIN:
        if (dtype == DT_INT32)
            return run_batched<MinI32>(in, out, rows, cols, excl, kind, s);
        if (dtype == DT_UINT32)
            return run_batched<MinU32>(in, out, rows, cols, excl, kind, s);
        return run_batched<MinF32>(in, out, rows, cols, excl, kind, s);
    case OP_AND:
        return run_batched<AndU32>(in, out, rows, cols, excl, kind, s);
    case OP_OR:
        return run_batched<OrU32>(in, out, rows, cols, excl, kind, s);
    case OP_PROD:
        if (dtype == DT_FLOAT32)
            return run_batched<MulF32>(in, out, rows, cols, excl, kind, s);
        return run_batched<MulU32>(in, out, rows, cols, excl, kind, s);
    case OP_AFFINE:
        return run_batched<AffU32>(in, out, rows, cols, excl, kind, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ls
