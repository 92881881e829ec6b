// ls_sort.hip -- stable LSD radix sort of 32-bit keys on the scan (gfx950).
//
// The application of scan that the pages cite most: a radix sort places every key
// of one digit value by the scan of that digit's predicate, with the second
// group offset by the size of the first, so that each pass is stable and needs
// no comparisons (geek-doc.cn parallel prefix scan page, section 一); with
// several bits per pass this becomes per-digit histograms, a prefix sum over
// them, and a reordering (lpnh.cn parallel scan overview, section 4.2).
//
// Here: four passes of 8-bit digits, least significant first.  Each pass is
//   1. histogram: every wave owns a tile of RS_TILE consecutive keys and counts
//      its digits in LDS; counts go to hist[digit * tiles + tile] (digit-major);
//   2. the library's own single-pass exclusive scan over hist -- after it,
//      hist[d * tiles + t] is where tile t's first key of digit d goes;
//   3. scatter: each wave walks its tile in input order, 64 keys at a time, and
//      ranks each key among the equal digits of that group with 8 ballots (one
//      per digit bit); per-digit cursors in LDS carry the ranks across groups.
//      Equal keys keep their order: the pass is stable, so the sort is.
// Keys are compared in their type's order through an order-preserving map to
// unsigned integers (int32: sign bit flipped; float32: IEEE total order).
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

constexpr int RS_BLOCK = 256;  // four independent waves
constexpr int RS_WAVES = RS_BLOCK / 64;
constexpr int RS_ITEMS = 16;   // keys per lane per tile
constexpr int RS_TILE = 64 * RS_ITEMS;  // 1024 keys per wave tile
constexpr int RS_BITS = 8;
constexpr int RS_DIGITS = 1 << RS_BITS;
constexpr int RS_PASSES = 32 / RS_BITS;

template <int DT>
__device__ __forceinline__ uint32_t order_key(uint32_t k)
{
    if constexpr (DT == DT_INT32)
        return k ^ 0x80000000u;
    else if constexpr (DT == DT_FLOAT32)
        return (k & 0x80000000u) ? ~k : (k | 0x80000000u);
    else
        return k;
}

// Key i of lane l in wave tile t: element t*RS_TILE + i*64 + l, so each group of
// 64 keys is one coalesced 256-byte load and groups come in input order.
template <int DT>
__global__ __launch_bounds__(RS_BLOCK) void rs_hist_kernel(const uint32_t* __restrict__ keys, int64_t n,
                                                           int shift, uint32_t* __restrict__ hist,
                                                           int64_t tiles)
{
    __shared__ uint32_t cnt[RS_WAVES][RS_DIGITS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile = int64_t(blockIdx.x) * RS_WAVES + wave;
    if (tile >= tiles)
        return;  // waves are independent: no block barrier below
#pragma unroll
    for (int q = 0; q < RS_DIGITS / 64; ++q)
        cnt[wave][lane * (RS_DIGITS / 64) + q] = 0;
    const int64_t base = tile * RS_TILE;
    const int64_t rem = n - base;
    const uint32_t valid = rem < RS_TILE ? uint32_t(rem) : uint32_t(RS_TILE);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(keys + base, valid * 4u);
    uint32_t k[RS_ITEMS];
#pragma unroll
    for (int i = 0; i < RS_ITEMS; ++i)
        k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, uint32_t(i * 64 + lane) * 4u, 0, CACHE_NT);
#pragma unroll
    for (int i = 0; i < RS_ITEMS; ++i) {
        if (uint32_t(i * 64 + lane) < valid)
            atomicAdd(&cnt[wave][(order_key<DT>(k[i]) >> shift) & (RS_DIGITS - 1)], 1u);
    }
#pragma unroll
    for (int q = 0; q < RS_DIGITS / 64; ++q) {
        const int d = lane * (RS_DIGITS / 64) + q;
        hist[int64_t(d) * tiles + tile] = cnt[wave][d];
    }
}

template <int DT, bool VALS>
__global__ __launch_bounds__(RS_BLOCK) void rs_scatter_kernel(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin, uint32_t* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, const uint32_t* __restrict__ offs, int64_t tiles)
{
    __shared__ uint32_t pos[RS_WAVES][RS_DIGITS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t tile = int64_t(blockIdx.x) * RS_WAVES + wave;
    if (tile >= tiles)
        return;
#pragma unroll
    for (int q = 0; q < RS_DIGITS / 64; ++q) {
        const int d = lane * (RS_DIGITS / 64) + q;
        pos[wave][d] = offs[int64_t(d) * tiles + tile];
    }
    const int64_t base = tile * RS_TILE;
    const int64_t rem = n - base;
    const uint32_t valid = rem < RS_TILE ? uint32_t(rem) : uint32_t(RS_TILE);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kin + base, valid * 4u);
    uint32_t k[RS_ITEMS], v[RS_ITEMS];
#pragma unroll
    for (int i = 0; i < RS_ITEMS; ++i)
        k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, uint32_t(i * 64 + lane) * 4u, 0, CACHE_NT);
    if constexpr (VALS) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vin + base, valid * 4u);
#pragma unroll
        for (int i = 0; i < RS_ITEMS; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, uint32_t(i * 64 + lane) * 4u, 0, CACHE_NT);
    }
    const uint64_t below = (uint64_t(1) << lane) - 1;  // lanes before this one
#pragma unroll
    for (int i = 0; i < RS_ITEMS; ++i) {
        const bool live = uint32_t(i * 64 + lane) < valid;
        const uint32_t d = (order_key<DT>(k[i]) >> shift) & (RS_DIGITS - 1);
        // lanes of this group holding the same digit
        uint64_t peers = __ballot(live);
#pragma unroll
        for (int b = 0; b < RS_BITS; ++b) {
            const uint64_t ones = __ballot((d >> b) & 1u);
            peers &= ((d >> b) & 1u) ? ones : ~ones;
        }
        if (live) {
            const uint32_t rank = __builtin_popcountll(peers & below);
            const uint32_t p = pos[wave][d] + rank;
            kout[p] = k[i];
            if constexpr (VALS)
                vout[p] = v[i];
            if (rank == 0)  // the first lane of the group advances the digit's cursor
                pos[wave][d] += uint32_t(__builtin_popcountll(peers));
        }
    }
}

// ------------------------------------------------------------------ host side

static size_t rs_round(size_t b) { return (b + 255) & ~size_t(255); }
static int64_t rs_tiles(int64_t n) { return (n + RS_TILE - 1) / RS_TILE; }

size_t sort_workspace_bytes(int64_t n, bool with_values)
{
    const int64_t tiles = rs_tiles(n) < 1 ? 1 : rs_tiles(n);
    const int64_t m = int64_t(RS_DIGITS) * tiles;
    size_t b = rs_round(size_t(n) * 4);              // keys between passes
    if (with_values)
        b += rs_round(size_t(n) * 4);                // values between passes
    b += rs_round(size_t(m) * 4);                    // digit histogram / offsets
    b += scan_workspace_bytes(m, SCHEME_SINGLE_PASS); // its scan
    return b;
}

template <int DT>
static hipError_t run_sort(const uint32_t* kin, uint32_t* kout, const uint32_t* vin, uint32_t* vout,
                           int64_t n, char* ws, hipStream_t s)
{
    const int64_t tiles = rs_tiles(n);
    const int64_t m = int64_t(RS_DIGITS) * tiles;
    const bool vals = vin != nullptr;
    char* p = ws;
    uint32_t* tk = reinterpret_cast<uint32_t*>(p);
    p += rs_round(size_t(n) * 4);
    uint32_t* tv = nullptr;
    if (vals) {
        tv = reinterpret_cast<uint32_t*>(p);
        p += rs_round(size_t(n) * 4);
    }
    uint32_t* hist = reinterpret_cast<uint32_t*>(p);
    p += rs_round(size_t(m) * 4);
    void* scan_ws = p;
    const dim3 grid(static_cast<uint32_t>((tiles + RS_WAVES - 1) / RS_WAVES)), block(RS_BLOCK);
    const uint32_t* sk = kin;
    const uint32_t* sv = vin;
    for (int pass = 0; pass < RS_PASSES; ++pass) {
        const int shift = pass * RS_BITS;
        uint32_t* dk = (pass % 2 == 0) ? tk : kout;  // the last pass lands in kout
        uint32_t* dv = (pass % 2 == 0) ? tv : vout;
        hipLaunchKernelGGL((rs_hist_kernel<DT>), grid, block, 0, s, sk, n, shift, hist, tiles);
        hipError_t e = launch_scan(hist, hist, m, DT_UINT32, OP_SUM, false, nullptr, scan_ws,
                                   SCHEME_SINGLE_PASS, s);
        if (e != hipSuccess)
            return e;
        if (vals)
            hipLaunchKernelGGL((rs_scatter_kernel<DT, true>), grid, block, 0, s, sk, sv, dk, dv, n, shift,
                               hist, tiles);
        else
            hipLaunchKernelGGL((rs_scatter_kernel<DT, false>), grid, block, 0, s, sk, sv, dk, dv, n,
                               shift, hist, tiles);
        sk = dk;
        sv = dv;
    }
    return hipGetLastError();
}

hipError_t launch_sort(const void* keys_in, void* keys_out, const void* vals_in, void* vals_out, int64_t n,
                       int dtype, void* ws, hipStream_t s)
{
    if (n == 0)
        return hipSuccess;
    const auto* kin = reinterpret_cast<const uint32_t*>(keys_in);
    auto* kout = reinterpret_cast<uint32_t*>(keys_out);
    const auto* vin = reinterpret_cast<const uint32_t*>(vals_in);
    auto* vout = reinterpret_cast<uint32_t*>(vals_out);
    char* w = reinterpret_cast<char*>(ws);
    switch (dtype) {
    case DT_INT32: return run_sort<DT_INT32>(kin, kout, vin, vout, n, w, s);
    case DT_UINT32: return run_sort<DT_UINT32>(kin, kout, vin, vout, n, w, s);
    default: return run_sort<DT_FLOAT32>(kin, kout, vin, vout, n, w, s);
    }
}

}  // namespace ls
