// lse.hip -- max/sum-aware LSE pack and stable LSE-weighted combine for
// decode/context-parallel attention (vllm-ascend "[Performance][Attention]
// Fuse local SFA LSE formation into DCP pack": the pack forms
// LSE = softmax_max + log(softmax_sum) while writing the packed exchange
// layout, invalid statistics give a -inf contribution, and the stable combine
// consumes the received partials).
//
// Design for gfx950.  Both kernels are HBM-bound (about one flop per byte), so
// the work is laid out for memory: payload rows move as 16-byte vectors with
// several requests in flight per lane; the per-row statistics are handled by a
// group of G lanes (G >= P, a power of two <= 64) that reduces the P partial
// LSEs with cross-lane shuffles, so each partial's exp is taken once and the O
// rows of invalid partials are never fetched.  No MFMA: nothing here is a
// dense contraction.
#include "cam_device.h"

namespace cam {

// ---------------------------------------------------------------------------
// Pack
// ---------------------------------------------------------------------------

// (t, h) of row q of chunk (p, r): scatter over heads keeps every token and
// head block r; scatter over tokens keeps every head and token block r.
__device__ __forceinline__ void pack_row_th(const Pack& a, uint32_t r, uint32_t q, uint64_t& t,
                                            uint64_t& h)
{
    const uint32_t outer = fdiv(q, a.div_inner);
    const uint32_t in = q - outer * a.inner;
    if (a.scatter_heads) {
        t = outer;
        h = uint64_t(r) * a.Hp + in;
    } else {
        t = uint64_t(r) * a.Tp + outer;
        h = in;
    }
}

template <int W, bool GUARD>
__device__ __forceinline__ void pack_o_tile(const Pack& a, uint32_t r, const char* src, char* dst, uint32_t v0)
{
    typedef typename VecOf<W>::type V;
    V x[kVecsPerThread];
#pragma unroll
    for (int u = 0; u < kVecsPerThread; ++u) {
        const uint32_t v = v0 + uint32_t(u * kThreads);
        if (!GUARD || v < a.o_vecs) {
            const uint32_t q = fdiv(v, a.div_cv);
            const uint32_t k = v - q * a.cv;
            uint64_t t, h;
            pack_row_th(a, r, q, t, h);
            const int64_t off = int64_t(t) * a.o_st_b + int64_t(h) * a.o_sh_b + int64_t(k) * W;
            x[u] = *reinterpret_cast<const V*>(src + off);
        }
    }
#pragma unroll
    for (int u = 0; u < kVecsPerThread; ++u) {
        const uint32_t v = v0 + uint32_t(u * kThreads);
        if (!GUARD || v < a.o_vecs)
            st<W>(dst, v, x[u]);
    }
}

template <int W>
__global__ __launch_bounds__(kThreads) void k_pack(Pack a)
{
    const uint32_t n_total = a.n_o_tiles + a.n_l_tiles;
    for (uint32_t tile = blockIdx.x; tile < n_total; tile += gridDim.x) {
        if (tile < a.n_o_tiles) {
            // O-region: bit copy of the payload rows into chunk (p, r)
            const uint32_t chunk = fdiv(tile, a.div_otpc);
            const uint32_t ti = tile - chunk * a.o_tiles_per_chunk;
            const uint32_t p = fdiv(chunk, a.div_P);
            const uint32_t r = chunk - p * a.P;
            const char* src = static_cast<const char*>(a.out) + int64_t(p) * a.o_sp_b;
            char* dst = static_cast<char*>(a.packed) + uint64_t(chunk) * a.chunk_b;
            const uint32_t vt = ti * uint32_t(kTileVecs);
            if (vt + uint32_t(kTileVecs) <= a.o_vecs)
                pack_o_tile<W, false>(a, r, src, dst, vt + threadIdx.x);
            else
                pack_o_tile<W, true>(a, r, src, dst, vt + threadIdx.x);
        } else {
            // L-region: one row per lane, LSE formed from the statistics
            const uint32_t lt = tile - a.n_o_tiles;
            const uint32_t chunk = fdiv(lt, a.div_ltpc);
            const uint32_t ti = lt - chunk * a.l_tiles_per_chunk;
            const uint32_t p = fdiv(chunk, a.div_P);
            const uint32_t r = chunk - p * a.P;
            const uint32_t q = ti * uint32_t(kThreads) + threadIdx.x;
            if (q < a.rows) {
                uint64_t t, h;
                pack_row_th(a, r, q, t, h);
                const float m = a.smax[int64_t(p) * a.m_sp + int64_t(t) * a.m_st + int64_t(h) * a.m_sh];
                const float s = a.ssum[int64_t(p) * a.s_sp + int64_t(t) * a.s_st + int64_t(h) * a.s_sh];
                float lse = -__builtin_inff();
                // NaN fails every comparison, so "s > 0" also rejects a NaN sum
                if (__builtin_isfinite(m) && __builtin_isfinite(s) && s > 0.0f)
                    lse = float(double(m) + log(double(s)));
                float* l = reinterpret_cast<float*>(static_cast<char*>(a.packed) +
                                                    uint64_t(chunk) * a.chunk_b + a.o_region_b);
                l[q] = lse;
            }
        }
    }
}

cam_status launch_pack(const Pack& a, void* stream)
{
    const void* fn = nullptr;
    if (a.width == 16) fn = reinterpret_cast<const void*>(&k_pack<16>);
    if (a.width == 8) fn = reinterpret_cast<const void*>(&k_pack<8>);
    if (a.width == 4) fn = reinterpret_cast<const void*>(&k_pack<4>);
    if (a.width == 2) fn = reinterpret_cast<const void*>(&k_pack<2>);
    return launch(fn, a, uint64_t(a.n_o_tiles) + a.n_l_tiles, stream, "lse_pack");
}

// ---------------------------------------------------------------------------
// Combine
// ---------------------------------------------------------------------------

template <int W>
struct Halves {
    uint16_t h[W / 2];
};

template <bool FP16>
__device__ __forceinline__ float half_to_f32(uint16_t x)
{
    if (FP16)
        return float(__builtin_bit_cast(_Float16, x));
    return __uint_as_float(uint32_t(x) << 16);
}

template <bool FP16>
__device__ __forceinline__ uint16_t f32_to_half(float f)
{
    if (FP16)
        return __builtin_bit_cast(uint16_t, _Float16(f));
    return uint16_t(f32_to_bf16_bits(f));
}

// Causal admission of KV piece p for the token t of a packed THD batch: the
// piece must be non-empty and start at or before t's position in its sequence.
__device__ __forceinline__ bool causal_piece_ok(const int32_t* cu, int32_t nseq, uint32_t P,
                                                uint32_t p, uint32_t t)
{
    int32_t lo = 0, hi = nseq;
    while (hi - lo > 1) {
        const int32_t mid = (lo + hi) >> 1;
        if (int64_t(cu[mid]) <= int64_t(t))
            lo = mid;
        else
            hi = mid;
    }
    const int64_t c0 = cu[lo];
    const int64_t L = int64_t(cu[lo + 1]) - c0;
    const int64_t k = int64_t(t) - c0;
    if (k < 0 || k >= L)
        return false;
    const int64_t start = (int64_t(p) * L) / P;
    const int64_t end = (int64_t(p + 1) * L) / P;
    return start < end && start <= k;
}

// Number of partial rows fetched together: the valid partials of a row are
// compacted and loaded CH at a time with no branch between the loads (a short
// last batch repeats its last valid row with weight 0, so an invalid partial's
// row is never touched).
#ifndef CAM_COMBINE_BATCH
#define CAM_COMBINE_BATCH 8
#endif
constexpr int kCombineBatch = CAM_COMBINE_BATCH;

template <int W, bool FP16, bool VARLEN>
__global__ __launch_bounds__(kThreads) void k_combine(Combine a)
{
    typedef typename VecOf<W>::type V;
    constexpr int E = W / 2;  // payload elements per vector
    constexpr int CH = kCombineBatch;

    const uint32_t G = 1u << a.g_log2;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t gl = lane & (G - 1u);      // lane within the row group
    const uint32_t gbase = lane & ~(G - 1u);  // first lane of the group in the wave
    const uint64_t gmask = G == 64u ? ~0ull : ((1ull << G) - 1ull);
    const uint32_t rows_per_block = kThreads >> a.g_log2;

    for (uint64_t rb = uint64_t(blockIdx.x) * rows_per_block; rb < a.n_rows;
         rb += uint64_t(gridDim.x) * rows_per_block) {
        const uint64_t row = rb + (threadIdx.x >> a.g_log2);
        const bool active = row < a.n_rows;
        uint32_t t = 0, h = 0;
        if (active) {
            t = fdiv(uint32_t(row), a.div_H);
            h = uint32_t(row) - t * a.H;
        }
        // statistics: lane gl of the group owns partial gl
        bool valid = false;
        float L = -__builtin_inff();
        if (active && gl < a.P) {
            bool admitted = true;
            if (VARLEN)
                admitted = causal_piece_ok(a.cu, a.nseq, a.P, gl, t);
            if (admitted) {
                L = a.pl[int64_t(gl) * a.pl_sp + int64_t(t) * a.pl_st + int64_t(h) * a.pl_sh];
                valid = __builtin_isfinite(L);
            }
        }
        float M = valid ? L : -__builtin_inff();
        for (uint32_t off = G >> 1; off > 0; off >>= 1)
            M = fmaxf(M, __shfl_xor(M, int(off), int(G)));
        const uint64_t vmask = (__ballot(valid) >> gbase) & gmask;
        const float w = valid ? expf(L - M) : 0.0f;
        float Z = w;
        for (uint32_t off = G >> 1; off > 0; off >>= 1)
            Z += __shfl_xor(Z, int(off), int(G));
        if (!active)
            continue;

        char* orow = static_cast<char*>(a.out) + int64_t(t) * a.o_st_b + int64_t(h) * a.o_sh_b;
        if (vmask == 0) {
            // no valid partial: +0 everywhere, -inf LSE
            Halves<W> zh;
#pragma unroll
            for (int e = 0; e < E; ++e)
                zh.h[e] = 0;
            const V zero = __builtin_bit_cast(V, zh);
            for (uint32_t k = gl; k < a.cv; k += G)
                *reinterpret_cast<V*>(orow + int64_t(k) * W) = zero;
            if (gl == 0 && a.lse_out)
                a.lse_out[int64_t(t) * a.lo_st + int64_t(h) * a.lo_sh] = -__builtin_inff();
            continue;
        }
        const float invZ = 1.0f / Z;
        const char* prow = static_cast<const char*>(a.po) + int64_t(t) * a.po_st_b + int64_t(h) * a.po_sh_b;
        // Every lane of the group runs every iteration, so the weight shuffles
        // below always read active lanes; a lane past the row's last vector
        // re-reads the last vector (a valid address) and stores nothing.
        for (uint32_t kb = 0; kb < a.cv; kb += G) {
            const uint32_t k = kb + gl < a.cv ? kb + gl : a.cv - 1;
            float acc[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] = 0.0f;
            const char* pk = prow + int64_t(k) * W;
            uint64_t m = vmask;
            while (m) {
                int idx[CH];
                float wv[CH];
                int last = 0;
#pragma unroll
                for (int u = 0; u < CH; ++u) {
                    const bool take = m != 0;
                    const int p = take ? __builtin_ctzll(m) : last;
                    m = take ? (m & (m - 1)) : m;
                    idx[u] = p;
                    last = p;
                    const float wp = __shfl(w, int(gbase + uint32_t(p)), 64);
                    wv[u] = take ? wp : 0.0f;
                }
                V x[CH];
#pragma unroll
                for (int u = 0; u < CH; ++u)
                    x[u] = *reinterpret_cast<const V*>(pk + int64_t(idx[u]) * a.po_sp_b);
#pragma unroll
                for (int u = 0; u < CH; ++u) {
                    const Halves<W> xh = __builtin_bit_cast(Halves<W>, x[u]);
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        acc[e] = fmaf(wv[u], half_to_f32<FP16>(xh.h[e]), acc[e]);
                }
            }
            if (kb + gl < a.cv) {
                Halves<W> oh;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    oh.h[e] = f32_to_half<FP16>(acc[e] * invZ);
                *reinterpret_cast<V*>(orow + int64_t(k) * W) = __builtin_bit_cast(V, oh);
            }
        }
        if (gl == 0 && a.lse_out)
            a.lse_out[int64_t(t) * a.lo_st + int64_t(h) * a.lo_sh] = M + logf(Z);
    }
}

cam_status launch_combine(const Combine& a, void* stream)
{
    const void* fn = nullptr;
#define CAM_PICK(Wd)                                                                            \
    if (a.width == Wd) {                                                                        \
        if (a.cu)                                                                               \
            fn = a.fp16 ? reinterpret_cast<const void*>(&k_combine<Wd, true, true>)            \
                        : reinterpret_cast<const void*>(&k_combine<Wd, false, true>);          \
        else                                                                                    \
            fn = a.fp16 ? reinterpret_cast<const void*>(&k_combine<Wd, true, false>)           \
                        : reinterpret_cast<const void*>(&k_combine<Wd, false, false>);         \
    }
    CAM_PICK(16) CAM_PICK(8) CAM_PICK(4) CAM_PICK(2)
#undef CAM_PICK
    const uint64_t rows_per_block = uint64_t(kThreads) >> a.g_log2;
    return launch(fn, a, (a.n_rows + rows_per_block - 1) / rows_per_block, stream, "lse_combine");
}

}  // namespace cam
