// relayout.hip -- Ulysses all-to-all relayout between sequence-sharded and
// head-sharded slabs of P logical ranks held in one GPU's HBM (FastVideo
// "[perf] Probe H3 chunked all-to-all with direct output slices":
// all_to_all_4D(x, 2, 1) and its inverse (1, 2), the fused kernel writing
// straight into the output slices), plus the cu_seqlens varlen form (cuLA
// "packed hybrid runtime and THD planner": packed THD batches).
//
// Design for gfx950.  The relayout is a pure permutation of runs of
// (H/P)*D elements that are contiguous on both sides (>= 512 bytes at the
// workloads here), so every wavefront access is already a coalesced run of
// 64 x W bytes; nothing needs an LDS transpose.  Each thread moves
// a few W-byte vectors (kDenseVecs, kVarlenVecs): all loads are issued before
// any store so that several 16-byte requests per lane are in flight, which is
// what keeps HBM3E busy on a streaming kernel.  Work is cut into tiles of
// kThreads times that many vectors inside a slab (dense) or plane (varlen);
// one division by the run length per vector (a multiply-high) recovers the
// row, everything else is per tile.
#include "cam_device.h"

namespace cam {

// Move one tile of a dense slab: vectors v0 + u*kThreads, u < kDenseVecs.
// GUARD = false is the straight-line path for tiles that lie wholly inside the
// slab: every load is issued before any store and no branch separates them,
// so each lane keeps kDenseVecs requests in flight.
template <int W, bool S2H, bool GUARD, int NTP>
__device__ __forceinline__ void dense_tile(const DenseRelayout& a, uint64_t head_base, uint64_t seq_base,
                                           uint32_t v0)
{
    typedef typename VecOf<W>::type V;
    V x[kDenseVecs];
    uint64_t dst_off[kDenseVecs];
#pragma unroll
    for (int u = 0; u < kDenseVecs; ++u) {
        const uint32_t v = v0 + uint32_t(u * kThreads);
        if (!GUARD || v < a.slab_vecs) {
            const uint32_t s = fdiv(v, a.div_c);
            const uint32_t k = v - s * a.c;
            const uint64_t so = seq_base + uint64_t(s) * a.Pc + k;
            const uint64_t ho = head_base + v;
            x[u] = ld<W, (NTP & 1) != 0>(a.src, S2H ? so : ho);
            dst_off[u] = S2H ? ho : so;
        }
    }
    issue_fence();
#pragma unroll
    for (int u = 0; u < kDenseVecs; ++u) {
        const uint32_t v = v0 + uint32_t(u * kThreads);
        if (!GUARD || v < a.slab_vecs)
            st<W, (NTP & 2) != 0>(a.dst, dst_off[u], x[u]);
    }
}

template <int W, bool S2H>
__global__ __launch_bounds__(kThreads) void k_dense_relayout(DenseRelayout a)
{
    constexpr bool XCD = S2H ? CAM_XCD_SEQ_TO_HEAD : CAM_XCD_HEAD_TO_SEQ;
    const uint32_t first = XCD ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    for (uint32_t tile = first; tile < a.n_tiles; tile += gridDim.x) {
        const uint32_t slab = fdiv(tile, a.div_tps);
        const uint32_t ti = tile - slab * a.tiles_per_slab;
        const uint32_t rb = fdiv(slab, a.div_P);
        const uint32_t j = slab - rb * a.P;
        const uint32_t r = fdiv(rb, a.div_B);
        const uint32_t b = rb - r * a.B;
        const uint64_t head_base = uint64_t(slab) * a.slab_vecs;
        const uint64_t seq_base = (uint64_t(j * a.B + b) * a.Sp * a.P + r) * a.c;
        const uint32_t vt = ti * uint32_t(kDenseTileVecs);
        constexpr int NTP = S2H ? CAM_NT_SEQ_TO_HEAD : CAM_NT_HEAD_TO_SEQ;
        if (vt + uint32_t(kDenseTileVecs) <= a.slab_vecs)
            dense_tile<W, S2H, false, NTP>(a, head_base, seq_base, vt + threadIdx.x);
        else
            dense_tile<W, S2H, true, NTP>(a, head_base, seq_base, vt + threadIdx.x);
    }
}

// Sequence-side vector offset of token t's row (i: t's sequence) for
// destination head block r of plane b, or -1 if the plan does not place t
// inside the buffer.
__device__ __forceinline__ int64_t varlen_seq_row(const VarlenRelayout& a, const int32_t* cu, int32_t i, uint32_t t,
                                                  uint32_t r, uint32_t b)
{
    const int64_t c0 = cu[i];
    const int64_t L = int64_t(cu[i + 1]) - c0;
    const int64_t k = int64_t(t) - c0;
    if (k < 0 || k >= L)
        return -1;
    const uint32_t p = piece_owner(uint32_t(k), uint32_t(L), a.div_P);
    const int64_t start = piece_start(p, uint32_t(L), a.div_P);
    const int64_t l = int64_t(a.rank_cu[int64_t(p) * (a.nseq + 1) + i]) + (k - start);
    const int64_t R = a.rank_off[p];
    const int64_t Tp = a.rank_off[p + 1] - R;
    if (l < 0 || l >= Tp)
        return -1;
    const int64_t row = int64_t(a.B) * R + int64_t(b) * Tp + l;
    if (row < 0 || row >= int64_t(a.B) * int64_t(a.T))
        return -1;
    return row * int64_t(a.Pc) + int64_t(r) * a.c;
}

// The same for a THD layout plan: cu holds the spans' first tokens (s: t's
// span).
__device__ __forceinline__ int64_t span_seq_row(const VarlenRelayout& a, const int32_t* cu, int32_t s, uint32_t t,
                                                uint32_t r, uint32_t b)
{
    const int64_t c0 = cu[s];
    const int64_t k = int64_t(t) - c0;
    if (k < 0 || k >= int64_t(cu[s + 1]) - c0)
        return -1;
    const uint32_t p = uint32_t(a.span_rank[s]);
    if (p >= a.P)
        return -1;
    const int64_t l = int64_t(a.span_local[s]) + k;
    const int64_t R = a.rank_off[p];
    const int64_t Tp = a.rank_off[p + 1] - R;
    if (l < 0 || l >= Tp)
        return -1;
    const int64_t row = int64_t(a.B) * R + int64_t(b) * Tp + l;
    if (row < 0 || row >= int64_t(a.B) * int64_t(a.T))
        return -1;
    return row * int64_t(a.Pc) + int64_t(r) * a.c;
}

template <bool SPANS>
__device__ __forceinline__ int64_t seq_row(const VarlenRelayout& a, const int32_t* cu, int32_t i, uint32_t t,
                                           uint32_t r, uint32_t b)
{
    return SPANS ? span_seq_row(a, cu, i, t, r, b) : varlen_seq_row(a, cu, i, t, r, b);
}

template <int W, bool S2H, bool GUARD, int NTP>
__device__ __forceinline__ void varlen_tile(const VarlenRelayout& a, const int64_t* row_off, uint64_t head_base,
                                            uint32_t vb, uint32_t ve, uint32_t row0)
{
    typedef typename VecOf<W>::type V;
    V x[kVarlenVecs];
    uint64_t dst_off[kVarlenVecs];
    bool live[kVarlenVecs];
#pragma unroll
    for (int u = 0; u < kVarlenVecs; ++u) {
        const uint32_t v = vb + threadIdx.x + uint32_t(u * kThreads);
        live[u] = !GUARD || v < ve;
        if (live[u]) {
            const uint32_t t = fdiv(v, a.div_c);
            const uint32_t k = v - t * a.c;
            const int64_t base = row_off[t - row0];
            live[u] = !GUARD || base >= 0;
            if (live[u]) {
                const uint64_t so = uint64_t(base) + k;
                const uint64_t ho = head_base + v;
                x[u] = ld<W, (NTP & 1) != 0>(a.src, S2H ? so : ho);
                dst_off[u] = S2H ? ho : so;
            }
        }
    }
    issue_fence();
#pragma unroll
    for (int u = 0; u < kVarlenVecs; ++u)
        if (live[u])
            st<W, (NTP & 2) != 0>(a.dst, dst_off[u], x[u]);
}

template <int W, bool S2H, bool SPANS>
__global__ __launch_bounds__(kThreads) void k_varlen_relayout(VarlenRelayout a)
{
    // sequence-side offset of every row the tile touches (a tile spans at most
    // kVarlenTileVecs + 1 rows when rows are one vector long)
    __shared__ int64_t row_off[kVarlenTileVecs + 1];
    __shared__ int32_t cu_lds[kCuCache];
    const bool cached = a.nseq < kCuCache;
    if (cached)  // visible after the barrier that opens every tile
        for (uint32_t i = threadIdx.x; i <= uint32_t(a.nseq); i += kThreads)
            cu_lds[i] = a.cu[i];
    constexpr bool XCD = S2H ? CAM_XCD_VARLEN_SEQ_TO_HEAD : CAM_XCD_VARLEN_HEAD_TO_SEQ;
    const uint32_t first = XCD ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    for (uint32_t tile = first; tile < a.n_tiles; tile += gridDim.x) {
        const uint32_t plane = fdiv(tile, a.div_tpp);
        const uint32_t ti = tile - plane * a.tiles_per_plane;
        const uint32_t r = fdiv(plane, a.div_B);
        const uint32_t b = plane - r * a.B;
        const uint64_t head_base = uint64_t(plane) * a.plane_vecs;
        const uint32_t vb = ti * uint32_t(kVarlenTileVecs);
        const uint64_t ve64 = uint64_t(vb) + kVarlenTileVecs;
        const uint32_t ve = uint32_t(ve64 < a.plane_vecs ? ve64 : a.plane_vecs);
        const uint32_t row0 = fdiv(vb, a.div_c);
        const uint32_t nrows = fdiv(ve - 1, a.div_c) - row0 + 1;
        __syncthreads();  // the previous tile's readers are done with row_off
        bool rows_ok = true;
        for (uint32_t i0 = 0; i0 < nrows; i0 += kThreads) {
            const uint32_t i = i0 + threadIdx.x;
            const bool live = i < nrows;
            const uint32_t t = row0 + i;
            // the row's sequence: from the LDS table, or else the wave finds
            // its first row's sequence in global memory with 64-wide probes
            // and each lane gallops from there
            int32_t sq;
            if (cached) {
                sq = live ? seq_of_token(cu_lds, a.nseq, t) : 0;
            } else {
                const uint32_t w0 = i0 + (threadIdx.x & ~63u);
                const int32_t hint = w0 < nrows ? wave_seq_of_token(a.cu, a.nseq, row0 + w0) : 0;
                sq = live ? seq_of_token_from(a.cu, a.nseq, hint, t) : 0;
            }
            if (live) {
                // the two calls differ only in the address space of the table,
                // so each compiles to plain LDS or global loads
                const int64_t off = cached ? seq_row<SPANS>(a, cu_lds, sq, t, r, b)
                                           : seq_row<SPANS>(a, a.cu, sq, t, r, b);
                row_off[i] = off;
                rows_ok = rows_ok && off >= 0;
            }
        }
        // full tile whose every row the plan places inside the buffer: no guards
        const bool fast = __syncthreads_and(rows_ok && ve - vb == uint32_t(kVarlenTileVecs));
        constexpr int NTP = S2H ? CAM_NT_VARLEN_SEQ_TO_HEAD : CAM_NT_VARLEN_HEAD_TO_SEQ;
        if (fast)
            varlen_tile<W, S2H, false, NTP>(a, row_off, head_base, vb, ve, row0);
        else
            varlen_tile<W, S2H, true, NTP>(a, row_off, head_base, vb, ve, row0);
    }
}

template <bool GUARD>
__device__ __forceinline__ void copy_tile(const Copy& a, uint64_t v0)
{
    typedef typename VecOf<16>::type V;
    V x[kCopyVecs];
#pragma unroll
    for (int u = 0; u < kCopyVecs; ++u) {
        const uint64_t v = v0 + uint64_t(u * kThreads);
        if (!GUARD || v < a.n_vecs)
            x[u] = ld<16, (CAM_NT_COPY & 1) != 0>(a.src, v);
    }
    issue_fence();
#pragma unroll
    for (int u = 0; u < kCopyVecs; ++u) {
        const uint64_t v = v0 + uint64_t(u * kThreads);
        if (!GUARD || v < a.n_vecs)
            st<16, (CAM_NT_COPY & 2) != 0>(a.dst, v, x[u]);
    }
}

__global__ __launch_bounds__(kThreads) void k_copy16(Copy a)
{
    const uint64_t n_tiles = (a.n_vecs + kCopyTileVecs - 1) / kCopyTileVecs;
    const uint64_t first = CAM_XCD_COPY ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    for (uint64_t tile = first; tile < n_tiles; tile += gridDim.x) {
        const uint64_t vt = tile * kCopyTileVecs;
        if (vt + kCopyTileVecs <= a.n_vecs)
            copy_tile<false>(a, vt + threadIdx.x);
        else
            copy_tile<true>(a, vt + threadIdx.x);
    }
}

// LDS-staged seq->head (ablation).  Loads: the tile's R*P*c vectors are one
// contiguous range of the source slab; each thread loads its share into
// registers (all loads issued first), writes them to LDS, and after the
// barrier every thread reads the vectors of its output positions from LDS:
// output position v = r*(R*c) + s*c + k (head block r, row s, vector k) is
// contiguous per r in the destination, and sits at LDS index s*P*c + r*c + k.
constexpr int kLdsVecsPerThread = 24;  // R*P*c <= 256 * 24 (checked on the host)

template <bool FULL>
__device__ __forceinline__ void lds_tile(const DenseLds& a, const u32x4* src, u32x4* lds, uint32_t rows,
                                         uint64_t dst_row0)
{
    constexpr bool NTL = (CAM_NT_SEQ_TO_HEAD & 1) != 0, NTS = (CAM_NT_SEQ_TO_HEAD & 2) != 0;
    const uint32_t n = rows * a.P * a.c;
    u32x4 x[kLdsVecsPerThread];
#pragma unroll
    for (int u = 0; u < kLdsVecsPerThread; ++u) {
        const uint32_t v = threadIdx.x + uint32_t(u) * kThreads;
        if (v < n)
            x[u] = ld_at<16, NTL>(src + v);
    }
    issue_fence();
#pragma unroll
    for (int u = 0; u < kLdsVecsPerThread; ++u) {
        const uint32_t v = threadIdx.x + uint32_t(u) * kThreads;
        if (v < n)
            lds[v] = x[u];
    }
    __syncthreads();
    const uint32_t rc = rows * a.c;
    for (uint32_t v = threadIdx.x; v < n; v += kThreads) {
        const uint32_t r = FULL ? fdiv(v, a.div_Rc) : v / rc;
        const uint32_t w = v - r * rc;
        const uint32_t srow = fdiv(w, a.div_c);
        const uint32_t k = w - srow * a.c;
        const u32x4 y = lds[srow * a.P * a.c + r * a.c + k];
        // head side: [P][B][S][c], row j*Sp + s0 + srow of head block r
        const uint64_t o = (uint64_t(r) * a.B * (a.Sp * a.P) + dst_row0 + srow) * a.c + k;
        st<16, NTS>(a.dst, o, y);
    }
}

__global__ __launch_bounds__(kThreads) void k_dense_s2h_lds(DenseLds a)
{
    extern __shared__ u32x4 lds[];
    for (uint32_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
        const uint32_t slab = fdiv(tile, a.div_tps);     // (j, b): source rank j, plane b
        const uint32_t ti = tile - slab * a.tiles_per_slab;
        const uint32_t j = fdiv(slab, a.div_B);
        const uint32_t b = slab - j * a.B;
        const uint64_t s0 = uint64_t(ti) * a.R;
        const uint32_t rows = uint32_t(a.Sp - s0 < a.R ? a.Sp - s0 : a.R);
        const u32x4* src = static_cast<const u32x4*>(a.src) + (uint64_t(slab) * a.Sp + s0) * a.P * a.c;
        // destination row of (b, j*Sp + s0) in head block 0: [P][B][S] rows
        const uint64_t dst_row0 = uint64_t(b) * (a.Sp * a.P) + uint64_t(j) * a.Sp + s0;
        __syncthreads();  // the previous tile's readers are done with LDS
        if (rows == a.R)
            lds_tile<true>(a, src, lds, rows, dst_row0);
        else
            lds_tile<false>(a, src, lds, rows, dst_row0);
    }
}

cam_status launch_dense_lds(const DenseLds& a, void* stream)
{
    return launch(reinterpret_cast<const void*>(&k_dense_s2h_lds), a, a.n_tiles, stream, "LDS-staged relayout",
                  uint64_t(a.R) * a.P * a.c * 16);
}

cam_status launch_dense_relayout(const DenseRelayout& a, void* stream)
{
    const void* fn = nullptr;
#define CAM_PICK(Wd)                                                                       \
    if (a.width == Wd)                                                                     \
        fn = a.seq_to_head ? reinterpret_cast<const void*>(&k_dense_relayout<Wd, true>)  \
                           : reinterpret_cast<const void*>(&k_dense_relayout<Wd, false>);
    CAM_PICK(16) CAM_PICK(8) CAM_PICK(4) CAM_PICK(2)
#undef CAM_PICK
    return launch(fn, a, a.n_tiles, stream, "dense relayout");
}

cam_status launch_varlen_relayout(const VarlenRelayout& a, void* stream)
{
    const void* fn = nullptr;
#define CAM_PICK(Wd)                                                                                    \
    if (a.width == Wd)                                                                                  \
        fn = a.spans ? (a.seq_to_head ? reinterpret_cast<const void*>(&k_varlen_relayout<Wd, true, true>)  \
                                      : reinterpret_cast<const void*>(&k_varlen_relayout<Wd, false, true>)) \
                     : (a.seq_to_head ? reinterpret_cast<const void*>(&k_varlen_relayout<Wd, true, false>) \
                                      : reinterpret_cast<const void*>(&k_varlen_relayout<Wd, false, false>));
    CAM_PICK(16) CAM_PICK(8) CAM_PICK(4) CAM_PICK(2)
#undef CAM_PICK
    return launch(fn, a, a.n_tiles, stream, "varlen relayout");
}

cam_status launch_copy(const Copy& a, void* stream)
{
    const uint64_t n_tiles = (a.n_vecs + kCopyTileVecs - 1) / kCopyTileVecs;
    return launch(reinterpret_cast<const void*>(&k_copy16), a, n_tiles, stream, "copy");
}

}  // namespace cam
