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
//     with a running carry across chunks.
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

template <class Op, bool EXCL, bool VEC>
__global__ __launch_bounds__(ROWB_BLOCK) void batched_block_kernel(const typename Op::T* in,
                                                                   typename Op::T* out, int64_t rows,
                                                                   int64_t cols)
{
    using T = typename Op::T;
    __shared__ T s_tot[2][ROWB_WAVES];
    const T id = Op::identity();
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
        const T* rin = in + row * cols;
        T* rout = out + row * cols;
        T carry = id;
        int par = 0;
        for (int64_t c0 = 0; c0 < cols; c0 += ROWB_CHUNK, par ^= 1) {
            const int64_t idx = c0 + 4 * int64_t(tid);
            Run4<T> r = load_run<T, VEC>(rin, idx, cols, id);
            r.v[1] = Op::apply(r.v[0], r.v[1]);
            r.v[2] = Op::apply(r.v[1], r.v[2]);
            r.v[3] = Op::apply(r.v[2], r.v[3]);
            const T inc = wave_inclusive_scan<Op>(r.v[3]);
            const T wex = wave_shift_up<Op>(inc);
            if (lane == 63)
                s_tot[par][wave] = inc;
            __syncthreads();
            T pre = id, agg = id;
#pragma unroll
            for (int ww = 0; ww < ROWB_WAVES; ++ww) {
                if (ww == wave)
                    pre = agg;
                agg = Op::apply(agg, s_tot[par][ww]);
            }
            const T cp = Op::apply(carry, Op::apply(pre, wex));
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
        // the next row reuses s_tot[0]: wait until every wave has read this row's totals
        __syncthreads();
    }
}

// ------------------------------------------------------------------ host side

template <class Op>
static hipError_t run_batched(const void* in, void* out, int64_t rows, int64_t cols, bool excl,
                              hipStream_t s)
{
    using T = typename Op::T;
    const T* pin = reinterpret_cast<const T*>(in);
    T* pout = reinterpret_cast<T*>(out);
    const bool vec = (((reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) & 15) == 0) &&
                     (cols % 4 == 0);
    if (cols <= 64) {
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
    const int64_t blocks = rows < max_grid ? rows : max_grid;
    const dim3 grid(static_cast<uint32_t>(blocks)), block(ROWB_BLOCK);
    if (excl) {
        if (vec)
            hipLaunchKernelGGL((batched_block_kernel<Op, true, true>), grid, block, 0, s, pin, pout, rows, cols);
        else
            hipLaunchKernelGGL((batched_block_kernel<Op, true, false>), grid, block, 0, s, pin, pout, rows, cols);
    } else {
        if (vec)
            hipLaunchKernelGGL((batched_block_kernel<Op, false, true>), grid, block, 0, s, pin, pout, rows, cols);
        else
            hipLaunchKernelGGL((batched_block_kernel<Op, false, false>), grid, block, 0, s, pin, pout, rows, cols);
    }
    return hipGetLastError();
}

hipError_t launch_batched(const void* in, void* out, int64_t rows, int64_t cols, int dtype, int op,
                          bool excl, hipStream_t s)
{
    if (rows == 0 || cols == 0)
        return hipSuccess;
    switch (op) {
    case OP_SUM:
        if (dtype == DT_FLOAT32)
            return run_batched<SumF32>(in, out, rows, cols, excl, s);
        return run_batched<SumU32>(in, out, rows, cols, excl, s);
    case OP_XOR:
        return run_batched<XorU32>(in, out, rows, cols, excl, s);
    case OP_MAX:
        if (dtype == DT_INT32)
            return run_batched<MaxI32>(in, out, rows, cols, excl, s);
        if (dtype == DT_UINT32)
            return run_batched<MaxU32>(in, out, rows, cols, excl, s);
        return run_batched<MaxF32>(in, out, rows, cols, excl, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace ls
