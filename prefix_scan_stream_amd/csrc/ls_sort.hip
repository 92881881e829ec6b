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
//   1. histogram: every block counts the digits of RS_HT tiles of RS_TILE
//      consecutive keys in LDS; counts go to hist[digit * tiles + tile]
//      (digit-major);
//   2. the library's own single-pass exclusive scan over hist -- after it,
//      hist[d * tiles + t] is where tile t's first key of digit d goes;
//   3. scatter: each wave walks its quarter of the tile in input order, 64 keys
//      at a time, and ranks each key among the equal digits of that group with
//      8 ballots (one per digit bit); per-digit cursors in LDS carry the ranks
//      across groups.  The block then groups its keys by digit in LDS and writes
//      each digit's run to consecutive output addresses.  Equal keys keep their
//      order: the pass is stable, so the sort is.
// Keys are compared in their type's order through an order-preserving map to
// unsigned integers (int32: sign bit flipped; float32: IEEE total order).
#include "ls_device.hpp"
#include "ls_internal.hpp"

namespace ls {

// 8-wave blocks, 8192-key tiles: longer digit runs per tile (32 keys on average)
// waste fewer partial-line writes in the scatter, and the LDS (43 / 76 KiB for
// keys / pairs) still allows 3 / 2 blocks per CU.  2^24 keys: 337-344 us against
// 367 us with 4096-key tiles, pairs 421-426 against 526-530 us; 16384-key tiles
// (one block per CU) are slower again (383 / 473-478 us).
#ifndef LS_RS_BLOCK
#define LS_RS_BLOCK 512
#endif
constexpr int RS_BLOCK = LS_RS_BLOCK;
constexpr int RS_WAVES = RS_BLOCK / 64;
constexpr int RS_ITEMS = 16;                   // keys per lane
constexpr int RS_WTILE = 64 * RS_ITEMS;        // 1024 keys per wave
constexpr int RS_TILE = RS_WAVES * RS_WTILE;   // 8192 keys per block tile
constexpr int RS_BITS = 8;
constexpr int RS_DIGITS = 1 << RS_BITS;
constexpr int RS_PASSES = 32 / RS_BITS;
static_assert(RS_BLOCK >= RS_DIGITS && RS_DIGITS % 64 == 0, "one thread per digit in the block-wide steps");
constexpr int RS_DWAVES = RS_DIGITS / 64;      // waves whose threads hold one digit each
constexpr int RS_XCDS = 8;                     // XCDs of an MI355X

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

template <int DT>
__device__ __forceinline__ uint32_t digit_of(uint32_t k, int shift)
{
    return (order_key<DT>(k) >> shift) & (RS_DIGITS - 1);
}

// Block tile t covers keys t*RS_TILE .. +RS_TILE-1; wave w of it the 1024 keys from
// w*RS_WTILE, key i of lane l at w*RS_WTILE + i*64 + l (a coalesced 256-byte load
// per group of 64, groups in input order).
//
// Histogram: one block counts RS_HT consecutive tiles (the next tile's keys load
// while the current one is counted) and writes each digit's RS_HT counts as one
// contiguous run.  One tile per block wrote each 4-byte count to its own line of
// the digit-major table, which cost 8x the table's bytes in HBM writes.
constexpr int RS_HT = 4;

// Block 0 also zeroes the workspace header and the `scan_tiles` status words of
// the scan that follows (a launch fewer per pass), so the sort needs nothing
// from its workspace's earlier contents.
template <int DT>
__global__ __launch_bounds__(RS_BLOCK) void rs_hist_kernel(const uint32_t* __restrict__ keys, int64_t n,
                                                           int shift, uint32_t* __restrict__ hist,
                                                           int64_t tiles, uint32_t* scan_hdr,
                                                           uint64_t* scan_status, int64_t scan_tiles)
{
    __shared__ uint32_t cnt[RS_HT][RS_DIGITS];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t t0 = int64_t(blockIdx.x) * RS_HT;
    if (blockIdx.x == 0) {
        // the header's ticket restarts; its error word (word 2) is kept, so that
        // ls_workspace_check still sees a give-up of an earlier pass
        if (tid < int(sizeof(WsHeader) / 4) && tid != 2)
            scan_hdr[tid] = 0u;
        for (int64_t i = tid; i < scan_tiles; i += RS_BLOCK) {
            scan_status[i * STATUS_STRIDE] = 0u;               // prefix word
            scan_status[i * STATUS_STRIDE + TOTAL_WORD] = 0u;  // total word
        }
    }
    for (int i = tid; i < RS_HT * RS_DIGITS; i += RS_BLOCK)
        cnt[i / RS_DIGITS][i % RS_DIGITS] = 0;

    // keys of the wave's part of tile t (elements past n are not counted)
    auto load = [&](int64_t t, uint32_t (&k)[RS_ITEMS]) -> uint32_t {
        const int64_t base = t * RS_TILE + int64_t(wave) * RS_WTILE;
        const int64_t rem = n - base;
        const uint32_t valid = rem <= 0 ? 0u : (rem < RS_WTILE ? uint32_t(rem) : uint32_t(RS_WTILE));
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(keys + (rem <= 0 ? 0 : base), valid * 4u);
#pragma unroll
        for (int i = 0; i < RS_ITEMS; ++i)
            k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, uint32_t(i * 64 + lane) * 4u, 0, CACHE_NT);
        return valid;
    };
    uint32_t ka[RS_ITEMS], kb[RS_ITEMS];
    uint32_t va = load(t0, ka), vb = 0;
    __syncthreads();
#pragma unroll
    for (int lt = 0; lt < RS_HT; ++lt) {
        uint32_t (&kc)[RS_ITEMS] = (lt & 1) ? kb : ka;
        uint32_t (&kn)[RS_ITEMS] = (lt & 1) ? ka : kb;
        const uint32_t vc = (lt & 1) ? vb : va;
        if (lt + 1 < RS_HT) {
            const uint32_t v = load(t0 + lt + 1, kn);  // tiles past the end load nothing
            if (lt & 1)
                va = v;
            else
                vb = v;
        }
#pragma unroll
        for (int i = 0; i < RS_ITEMS; ++i) {
            if (uint32_t(i * 64 + lane) < vc)
                atomicAdd(&cnt[lt][digit_of<DT>(kc[i], shift)], 1u);
        }
    }
    __syncthreads();
    // digit d's counts of tiles t0 .. t0 + RS_HT - 1 are consecutive words
    for (int i = tid; i < RS_HT * RS_DIGITS; i += RS_BLOCK) {
        const int d = i / RS_HT, lt = i % RS_HT;
        if (t0 + lt < tiles)
            hist[int64_t(d) * tiles + t0 + lt] = cnt[lt][d];
    }
}

// Stable scatter of one block tile:
//   1. each wave ranks its keys among equal digits in input order (8 ballots per
//      group of 64, a per-wave digit cursor in LDS) and ends with its digit counts;
//   2. one thread per digit: the block's digit runs (exclusive scan of the
//      per-digit totals over the block), each wave's offset inside its digit's
//      run, and the run's place in the output (the scanned histogram);
//   3. keys (and values) are staged in LDS grouped by digit, in input order
//      within a digit;
//   4. the staged tile is written out: consecutive positions of one digit go to
//      consecutive addresses, so runs of a digit are written together.
template <int DT, bool VALS>
__global__ __launch_bounds__(RS_BLOCK) void rs_scatter_kernel(
    const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin, uint32_t* __restrict__ kout,
    uint32_t* __restrict__ vout, int64_t n, int shift, const uint32_t* __restrict__ offs, int64_t tiles)
{
    __shared__ uint32_t s_keys[RS_TILE];
    __shared__ uint32_t s_vals[VALS ? RS_TILE : 1];
    __shared__ uint32_t wcnt[RS_WAVES][RS_DIGITS];   // per-wave digit counts, then offsets
    __shared__ uint32_t run_start[RS_DIGITS];        // where a digit's run starts in the tile
    __shared__ uint32_t run_dest[RS_DIGITS];         // where it goes in the output
    __shared__ uint32_t s_wtot[RS_WAVES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // Consecutive tiles on one XCD.  Tile t's run of a digit ends where tile t + 1's
    // run of it begins, so every run boundary is a memory sector written half by
    // one block and half by the next.  Blocks are dispatched to the eight XCDs
    // round-robin (block b to XCD b mod 8), each XCD with its own L2: with tile t on
    // block b, tile t + 1 on block b + 8, both halves of a boundary sector meet in
    // one L2 and go to HBM as one full write, where tiles on different XCDs cost a
    // read-modify-write of the sector at the memory.  MI355X, 2^24 keys: scatter
    // HBM traffic 1.22 -> 1.00 x the algorithmic bytes (keys), 1.16 -> 1.01
    // (pairs); pairs sort 378 -> 355 us.
    const int64_t per_xcd = (tiles + RS_XCDS - 1) / RS_XCDS;
    const int64_t tile = int64_t(blockIdx.x % RS_XCDS) * per_xcd + blockIdx.x / RS_XCDS;
    if (tile >= tiles)
        return;  // the grid is rounded up to a multiple of RS_XCDS

    for (int i = tid; i < RS_WAVES * RS_DIGITS; i += RS_BLOCK)
        wcnt[i / RS_DIGITS][i % RS_DIGITS] = 0;
    const int64_t tbase = tile * RS_TILE;
    const int64_t trem = n - tbase;
    const uint32_t tvalid = trem < RS_TILE ? uint32_t(trem) : uint32_t(RS_TILE);
    const int64_t base = tbase + int64_t(wave) * RS_WTILE;
    const int64_t rem = n - base;
    const uint32_t valid = rem <= 0 ? 0u : (rem < RS_WTILE ? uint32_t(rem) : uint32_t(RS_WTILE));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kin + (rem <= 0 ? 0 : base), valid * 4u);
    uint32_t k[RS_ITEMS], v[RS_ITEMS], rank[RS_ITEMS];
#pragma unroll
    for (int i = 0; i < RS_ITEMS; ++i)
        k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, uint32_t(i * 64 + lane) * 4u, 0, CACHE_NT);
    if constexpr (VALS) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vin + (rem <= 0 ? 0 : base), valid * 4u);
#pragma unroll
        for (int i = 0; i < RS_ITEMS; ++i)
            v[i] = __builtin_amdgcn_raw_buffer_load_b32(rv, uint32_t(i * 64 + lane) * 4u, 0, CACHE_NT);
    }
    const uint32_t d_me = tid;  // the digit this thread handles in the block-wide steps (tid < RS_DIGITS)
    // where this tile's run of digit d_me goes: one word per digit, each in its own
    // line (the table is digit-major), so it is read after the keys and written to
    // LDS only after the ranking.  Waiting for it before the ranking cost 3.4 us of
    // a 12.7 us tile (2^24 keys: 335-341 us against 345-347 us).
    const uint32_t my_dest = tid < RS_DIGITS ? offs[int64_t(d_me) * tiles + tile] : 0u;
    __syncthreads();

    // 1. rank inside the wave tile
    const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
    for (int i = 0; i < RS_ITEMS; ++i) {
        const bool live = uint32_t(i * 64 + lane) < valid;
        const uint32_t d = digit_of<DT>(k[i], shift);
        uint64_t peers = __ballot(live);
#pragma unroll
        for (int b = 0; b < RS_BITS; ++b) {
            const uint64_t ones = __ballot((d >> b) & 1u);
            peers &= ((d >> b) & 1u) ? ones : ~ones;
        }
        const uint32_t in_group = __builtin_popcountll(peers & below);
        const uint32_t before = live ? wcnt[wave][d] : 0u;
        rank[i] = before + in_group;
        if (live && in_group == 0)
            wcnt[wave][d] = before + uint32_t(__builtin_popcountll(peers));
    }
    if (tid < RS_DIGITS)
        run_dest[d_me] = my_dest;
    __syncthreads();

    // 2. per digit: offsets of the waves inside the digit's run, the run's start in
    // the tile (block-wide exclusive scan of the digit totals), its output place
    uint32_t tot = 0, inc = 0;
    if (wave < RS_DWAVES) {
#pragma unroll
        for (int w = 0; w < RS_WAVES; ++w) {
            const uint32_t c = wcnt[w][d_me];
            wcnt[w][d_me] = tot;
            tot += c;
        }
        inc = wave_inclusive_scan<SumU32>(tot);
        if (lane == 63)
            s_wtot[wave] = inc;
    }
    __syncthreads();
    if (wave < RS_DWAVES) {
        uint32_t wpre = 0;
#pragma unroll
        for (int w = 0; w < RS_DWAVES; ++w)
            wpre += (w < wave) ? s_wtot[w] : 0u;
        run_start[d_me] = wpre + inc - tot;
    }
    __syncthreads();

    // 3. stage grouped by digit
#pragma unroll
    for (int i = 0; i < RS_ITEMS; ++i) {
        if (uint32_t(i * 64 + lane) < valid) {
            const uint32_t d = digit_of<DT>(k[i], shift);
            const uint32_t q = run_start[d] + wcnt[wave][d] + rank[i];
            s_keys[q] = k[i];
            if constexpr (VALS)
                s_vals[q] = v[i];
        }
    }
    __syncthreads();

    // 4. write the digit runs
    for (uint32_t q = tid; q < tvalid; q += RS_BLOCK) {
        const uint32_t key = s_keys[q];
        const uint32_t d = digit_of<DT>(key, shift);
        const uint32_t dst = run_dest[d] + (q - run_start[d]);
        kout[dst] = key;
        if constexpr (VALS)
            vout[dst] = s_vals[q];
    }
}

// ------------------------------------------------------------------ host side

static size_t rs_round(size_t b) { return (b + 255) & ~size_t(255); }
static int64_t rs_tiles(int64_t n) { return (n + RS_TILE - 1) / RS_TILE; }

size_t sort_workspace_bytes(int64_t n, bool with_values)
{
    const int64_t tiles = rs_tiles(n) < 1 ? 1 : rs_tiles(n);
    const int64_t m = int64_t(RS_DIGITS) * tiles;
    size_t b = rs_round(scan_workspace_bytes(m, SCHEME_SINGLE_PASS));  // the histogram's scan, first
    b += rs_round(size_t(n) * 4);                    // keys between passes
    if (with_values)
        b += rs_round(size_t(n) * 4);                // values between passes
    b += rs_round(size_t(m) * 4);                    // digit histogram / offsets
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
    void* scan_ws = p;  // first: its header's error word is the workspace's (ls_workspace_check)
    auto* scan_status = reinterpret_cast<uint64_t*>(p + sizeof(WsHeader));
    p += rs_round(scan_workspace_bytes(m, SCHEME_SINGLE_PASS));
    uint32_t* tk = reinterpret_cast<uint32_t*>(p);
    p += rs_round(size_t(n) * 4);
    uint32_t* tv = nullptr;
    if (vals) {
        tv = reinterpret_cast<uint32_t*>(p);
        p += rs_round(size_t(n) * 4);
    }
    uint32_t* hist = reinterpret_cast<uint32_t*>(p);
    const int64_t scan_tiles = scan_sum_u32_tiles(m);  // status words the scan reads
    const dim3 grid(static_cast<uint32_t>((tiles + RS_XCDS - 1) / RS_XCDS * RS_XCDS)), block(RS_BLOCK);
    const dim3 hgrid(static_cast<uint32_t>((tiles + RS_HT - 1) / RS_HT));
    const uint32_t* sk = kin;
    const uint32_t* sv = vin;
    for (int pass = 0; pass < RS_PASSES; ++pass) {
        const int shift = pass * RS_BITS;
        uint32_t* dk = (pass % 2 == 0) ? tk : kout;  // the last pass lands in kout
        uint32_t* dv = (pass % 2 == 0) ? tv : vout;
        hipLaunchKernelGGL((rs_hist_kernel<DT>), hgrid, block, 0, s, sk, n, shift, hist, tiles,
                           reinterpret_cast<uint32_t*>(scan_ws), scan_status, scan_tiles);
        hipError_t e = launch_scan_sum_u32_excl(hist, hist, m, scan_ws, s);
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
