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
    V x[kPackVecs];
#pragma unroll
    for (int u = 0; u < kPackVecs; ++u) {
        const uint32_t v = v0 + uint32_t(u * kThreads);
        if (!GUARD || v < a.o_vecs) {
            const uint32_t q = fdiv(v, a.div_cv);
            const uint32_t k = v - q * a.cv;
            uint64_t t, h;
            pack_row_th(a, r, q, t, h);
            const int64_t off = int64_t(t) * a.o_st_b + int64_t(h) * a.o_sh_b + int64_t(k) * W;
            x[u] = ld_at<W, (CAM_NT_PACK & 1) != 0>(src + off);
        }
    }
    issue_fence();
#pragma unroll
    for (int u = 0; u < kPackVecs; ++u) {
        const uint32_t v = v0 + uint32_t(u * kThreads);
        if (!GUARD || v < a.o_vecs)
            st<W, (CAM_NT_PACK & 2) != 0>(dst, v, x[u]);
    }
}

template <int W>
__global__ __launch_bounds__(kThreads) void k_pack(Pack a)
{
    const uint32_t n_total = a.n_o_tiles + a.n_l_tiles;
    const uint32_t first = CAM_XCD_PACK ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    for (uint32_t tile = first; tile < n_total; tile += gridDim.x) {
        if (tile < a.n_o_tiles) {
            // O-region: bit copy of the payload rows into chunk (p, r)
            const uint32_t chunk = fdiv(tile, a.div_otpc);
            const uint32_t ti = tile - chunk * a.o_tiles_per_chunk;
            const uint32_t p = fdiv(chunk, a.div_P);
            const uint32_t r = chunk - p * a.P;
            const char* src = static_cast<const char*>(a.out) + int64_t(p) * a.o_sp_b;
            char* dst = static_cast<char*>(a.packed) + uint64_t(chunk) * a.chunk_b;
            const uint32_t vt = ti * uint32_t(kPackTileVecs);
            if (vt + uint32_t(kPackTileVecs) <= a.o_vecs)
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

// Causal admission of KV piece p for the token t of a packed THD batch (i:
// t's sequence): the piece must be non-empty and start at or before t's
// position in its sequence.
__device__ __forceinline__ bool causal_piece_ok(const int32_t* cu, int32_t i, const FastDiv& divP, uint32_t p,
                                                uint32_t t)
{
    const int64_t c0 = cu[i];
    const int64_t L = int64_t(cu[i + 1]) - c0;
    const int64_t k = int64_t(t) - c0;
    if (k < 0 || k >= L)
        return false;
    const uint32_t start = piece_start(p, uint32_t(L), divP);
    const uint32_t end = piece_start(p + 1, uint32_t(L), divP);
    return start < end && int64_t(start) <= k;
}

// Causal admission under a THD layout plan: partial p (rank p's KV) is
// admitted for the token at position k of sequence i iff rank p holds a
// position of sequence i at or before k, first[p][i] <= k (INT32_MAX when it
// holds none of the sequence).
__device__ __forceinline__ bool causal_span_ok(const int32_t* cu, int32_t nseq, const int32_t* first, int32_t i,
                                               uint32_t p, uint32_t t)
{
    const int64_t c0 = cu[i];
    const int64_t k = int64_t(t) - c0;
    if (k < 0 || k >= int64_t(cu[i + 1]) - c0)
        return false;
    return int64_t(first[int64_t(p) * nseq + i]) <= k;
}

// Which partials a token admits (a kernel template parameter, so each rule
// is its own kernel): every partial, the per-sequence piece rule over
// cu_seqlens, or a THD layout plan's first-position rule.
enum Causal : int { kAll = 0, kPieces = 1, kPlan = 2 };

template <int CZ, typename Rec>
__device__ __forceinline__ bool admitted_partial(const Rec& a, const int32_t* cu, int32_t i, uint32_t p, uint32_t t)
{
    if (CZ == kPlan)
        return causal_span_ok(cu, a.nseq, a.first, i, p, t);
    return causal_piece_ok(cu, i, a.div_P, p, t);
}

// The sequence of token t in a tile's phase 1, called by every lane of the
// wave: from the LDS copy of cu_seqlens when it is staged there; otherwise the
// wave first finds the sequence of its first row's token in global memory with
// 64-wide probes (every other lane's token is at or after it) and each lane
// gallops from there.  w_live: the wave's first row w_row exists.
template <typename Rec>
__device__ __forceinline__ int32_t tile_token_seq(const Rec& a, const int32_t* cu_lds, bool cached, bool w_live,
                                                  uint64_t w_row, bool live, uint32_t t)
{
    if (cached)
        return live ? seq_of_token(cu_lds, a.nseq, t) : 0;
    const int32_t hint = w_live ? wave_seq_of_token(a.cu, a.nseq, fdiv(uint32_t(w_row), a.div_H)) : 0;
    return live ? seq_of_token_from(a.cu, a.nseq, hint, t) : 0;
}

// Rank-major (sequence-sharded) row of token t of a packed THD batch: the
// row of the varlen relayout's sequence side for B = 1.
__device__ __forceinline__ int64_t varlen_token_row(const int32_t* cu, const Combine& a, int32_t i, uint32_t t)
{
    const uint32_t c0 = uint32_t(cu[i]);
    const uint32_t L = uint32_t(cu[i + 1]) - c0;
    const uint32_t k = t - c0;
    const uint32_t p = piece_owner(k, L, a.div_P);
    return a.rank_off[p] + int64_t(a.rank_cu[int64_t(p) * (a.nseq + 1) + i]) + (k - piece_start(p, L, a.div_P));
}

// Partial weights exp(L - M) <= 1 and their normaliser 1/Z.  The fast forms
// (hardware exp2 and reciprocal, about 1 ulp) are an option measured against
// the correctly rounded library calls.
#ifndef CAM_COMBINE_FAST_WEIGHTS
#define CAM_COMBINE_FAST_WEIGHTS 0
#endif
__device__ __forceinline__ float weight_exp(float x)
{
    if (CAM_COMBINE_FAST_WEIGHTS)
        return __expf(x);
    return expf(x);
}
__device__ __forceinline__ float recip(float z)
{
    if (CAM_COMBINE_FAST_WEIGHTS)
        return __builtin_amdgcn_rcpf(z);
    return 1.0f / z;
}

// The combine works on tiles of kCombineRows consecutive rows per workgroup.
// Phase 1 turns the tile's partial LSEs into weights in LDS: thread
// (row, p) loads one LSE (consecutive rows are consecutive addresses), a group
// of pow2(P) lanes reduces max and sum with shuffles, and the normalised
// weights, the validity mask and the output LSE go to LDS.  Phase 2 only
// streams payload: a group of G lanes covers one row (G 16-byte vectors at a
// time), keeps RF rows in flight, and loads each row's valid
// partials kCombineBatch at a time with no branch between the loads (a short
// batch repeats its last valid row with weight 0, so an invalid partial's row
// is never read).

__device__ __forceinline__ uint32_t uniform32(uint32_t x)
{
    return uint32_t(__builtin_amdgcn_readfirstlane(int(x)));
}
__device__ __forceinline__ uint64_t uniform64(uint64_t x)
{
    return uint64_t(uniform32(uint32_t(x))) | (uint64_t(uniform32(uint32_t(x >> 32))) << 32);
}

// The payload rows of a row's valid partials, in ascending order, as a
// compacted list built in phase 1: byte offsets from the partials' base and
// normalised weights.  N rows are loaded at once (N is exact, so no lane
// loads or accumulates a row it does not need), then accumulated in order.
template <int N, int W, bool FP16, bool NTL, int VPL>
__device__ __forceinline__ void combine_rows(const char* po, const int64_t* offs, const float* wks,
                                             const uint32_t (&kbyte)[VPL], float (&acc)[VPL][W / 2])
{
    typedef typename VecOf<W>::type V;
    constexpr int E = W / 2;
    int64_t o[N];
#pragma unroll
    for (int u = 0; u < N; ++u)
        o[u] = offs[u];
    V x[N][VPL];
#pragma unroll
    for (int u = 0; u < N; ++u)
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            x[u][v] = ld_at<W, NTL>(po + o[u] + kbyte[v]);
    issue_fence();
    float w[N];
#pragma unroll
    for (int u = 0; u < N; ++u)
        w[u] = wks[u];
#pragma unroll
    for (int u = 0; u < N; ++u)
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const Halves<W> xh = __builtin_bit_cast(Halves<W>, x[u][v]);
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[v][e] = fmaf(w[u], half_to_f32<FP16>(xh.h[e]), acc[v][e]);
        }
}

// E fp32 values rounded to the payload type (round to nearest even), packed
// as one access vector; bf16 pairs use the hardware's packed conversion.
template <int W, bool FP16>
__device__ __forceinline__ typename VecOf<W>::type round_payload(const float (&acc)[W / 2])
{
    constexpr int E = W / 2;
    Halves<W> oh;
    if constexpr (!FP16 && E % 2 == 0) {
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        struct Words {
            uint32_t w[E / 2];
        } words;
#pragma unroll
        for (int e = 0; e < E; e += 2) {
            const f2 v = {acc[e], acc[e + 1]};
            words.w[e / 2] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
        }
        return __builtin_bit_cast(typename VecOf<W>::type, words);
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            oh.h[e] = f32_to_half<FP16>(acc[e]);
        return __builtin_bit_cast(typename VecOf<W>::type, oh);
    }
}

// WAVE: one row group is a whole wave (rows of >= 64 vectors), so every
// per-row quantity of phase 2 is wave-uniform and is kept in scalar registers.
// OM: where the combined rows go -- 0 at the caller's strides, 1 token-major
// (head-scattered rows of the exchange), 2 rank-major (varlen sequence shards).
#ifdef CAM_COMBINE_WAVES_PER_EU
#define CAM_COMBINE_OCC __attribute__((amdgpu_waves_per_eu(CAM_COMBINE_WAVES_PER_EU)))
#else
#define CAM_COMBINE_OCC
#endif
template <int W, bool FP16, int CZ, int RF, bool WAVE, int OM>
__global__ __launch_bounds__(kThreads) CAM_COMBINE_OCC void k_combine(Combine a)
{
    typedef typename VecOf<W>::type V;
    constexpr int E = W / 2;  // payload elements per vector
    constexpr int CH = WAVE ? kCombineBatchWave : kCombineBatch;
    constexpr bool NTL = (CAM_NT_COMBINE & 1) != 0, NTS = (CAM_NT_COMBINE & 2) != 0;
    // per tile.  WAVE: weights [rows][P] by partial, validity masks, 1/Z.
    // Otherwise: each row's valid partials as a compacted list -- weights and
    // payload-row byte offsets [rows][P] (the first n of a row used) -- and
    // the row's count n.
    extern __shared__ float smem[];
    const uint32_t RB = a.rows_per_tile;
    float* w_lds = smem;                                                   // RB * P
    uint64_t* m_lds = reinterpret_cast<uint64_t*>(w_lds + ((RB * a.P + 1) & ~1u));  // WAVE: RB; else RB * P
    int64_t* q_lds = reinterpret_cast<int64_t*>(m_lds);                    // !WAVE: compacted offsets
    int64_t* o_lds = reinterpret_cast<int64_t*>(m_lds + (WAVE ? RB : RB * a.P));  // RB: output row offsets
    float* iz_lds = reinterpret_cast<float*>(o_lds + RB);                  // RB (WAVE: 1/Z; else the count)
    uint32_t* nv_lds = reinterpret_cast<uint32_t*>(iz_lds);
    int32_t* cu_lds = reinterpret_cast<int32_t*>(iz_lds + RB);             // nseq + 1 (varlen)
    const bool cached = CZ != kAll && a.nseq < kCuCache;
    if (cached)  // visible after the barrier that opens every tile
        for (uint32_t i = threadIdx.x; i <= uint32_t(a.nseq); i += blockDim.x)
            cu_lds[i] = a.cu[i];

    const uint32_t lane = threadIdx.x & 63u;
    // phase-1 geometry: GP lanes per row
    const uint32_t GP = 1u << a.gp_log2;
    const uint32_t sp = lane & (GP - 1u);
    const uint32_t sbase = lane & ~(GP - 1u);
    const uint64_t spmask = GP == 64u ? ~0ull : ((1ull << GP) - 1ull);
    // phase-2 geometry: G lanes per row
    const uint32_t G = 1u << a.g_log2;
    const uint32_t gl = lane & (G - 1u);
    const uint32_t nthr = blockDim.x;                           // 64, 128 or 256
    const uint32_t groups = nthr >> a.g_log2;                   // row groups per block
    const uint32_t group = threadIdx.x >> a.g_log2;

    const uint64_t first = a.xcd ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    for (uint64_t tile = first; tile < a.n_tiles; tile += gridDim.x) {
        const uint64_t row0 = tile * RB;
        // ---- phase 1: statistics of the tile's rows
        __syncthreads();  // the previous tile's readers are done with LDS
        for (uint32_t base = 0; base < RB * GP; base += nthr) {
            const uint32_t tau = base + threadIdx.x;
            const uint32_t rl = tau >> a.gp_log2;  // row within the tile
            const uint64_t row = row0 + rl;
            const bool live = rl < RB && row < a.n_rows;
            uint32_t t = 0, h = 0;
            if (live) {
                t = fdiv(uint32_t(row), a.div_H);
                h = uint32_t(row) - t * a.H;
            }
            int32_t seq = 0;  // the token's sequence (the causal rules and output mode 2)
            if (CZ != kAll) {
                const uint32_t wl = (base + (threadIdx.x & ~63u)) >> a.gp_log2;  // the wave's first row
                seq = tile_token_seq(a, cu_lds, cached, wl < RB && row0 + wl < a.n_rows, row0 + wl, live, t);
            }
            bool valid = false;
            float L = -__builtin_inff();
            if (live && sp < a.P) {
                bool admitted = true;
                if (CZ != kAll)
                    // the two calls differ only in the address space of the table
                    admitted = cached ? admitted_partial<CZ>(a, cu_lds, seq, sp, t)
                                      : admitted_partial<CZ>(a, a.cu, seq, sp, t);
                if (admitted) {
                    L = a.pl[int64_t(sp) * a.pl_sp + int64_t(t) * a.pl_st + int64_t(h) * a.pl_sh];
                    valid = __builtin_isfinite(L);
                }
            }
            float M = valid ? L : -__builtin_inff();
            for (uint32_t off = GP >> 1; off > 0; off >>= 1)
                M = fmaxf(M, __shfl_xor(M, int(off), int(GP)));
            const uint64_t vmask = (__ballot(valid) >> sbase) & spmask;
            const float w = valid ? weight_exp(L - M) : 0.0f;
            float Z = w;
            for (uint32_t off = GP >> 1; off > 0; off >>= 1)
                Z += __shfl_xor(Z, int(off), int(GP));
            if (live) {
                const float iz = vmask ? recip(Z) : 0.0f;
                if (WAVE) {
                    if (sp < a.P)
                        w_lds[rl * a.P + sp] = w * iz;
                } else if (valid) {
                    const uint32_t slot = uint32_t(__builtin_popcountll(vmask & ((1ull << sp) - 1ull)));
                    w_lds[rl * a.P + slot] = w * iz;
                    q_lds[rl * a.P + slot] =
                        int64_t(sp) * a.po_sp_b + int64_t(t) * a.po_st_b + int64_t(h) * a.po_sh_b;
                }
                if (sp == 0) {
                    int64_t o_off, l_off;
                    if (OM == 0) {
                        o_off = int64_t(t) * a.o_st_b + int64_t(h) * a.o_sh_b;
                        l_off = int64_t(t) * a.lo_st + int64_t(h) * a.lo_sh;
                    } else {
                        int64_t g;
                        if (OM == 1) {
                            const uint32_t tq = fdiv(h, a.div_Hp);
                            g = int64_t(tq) * a.Hq + int64_t(t) * a.Hp + (h - tq * a.Hp);
                        } else {
                            g = (cached ? varlen_token_row(cu_lds, a, seq, t) : varlen_token_row(a.cu, a, seq, t)) *
                                    a.H + h;
                        }
                        // a plan that places the token outside [0, T) skips the row
                        const bool in = g >= 0 && uint64_t(g) < a.n_rows;
                        o_off = in ? g * int64_t(a.o_row_b) : -1;
                        l_off = in ? g : -1;
                    }
                    if (WAVE) {
                        m_lds[rl] = vmask;
                        iz_lds[rl] = iz;
                    } else {
                        nv_lds[rl] = uint32_t(__builtin_popcountll(vmask));
                    }
                    o_lds[rl] = o_off;
                    if (a.lse_out && l_off >= 0)
                        a.lse_out[l_off] = vmask ? M + logf(Z) : -__builtin_inff();
                }
            }
        }
        __syncthreads();

        // ---- phase 2: stream the payload rows
        const uint64_t left = a.n_rows - row0;
        const uint32_t nr = left < RB ? uint32_t(left) : RB;  // rows of this tile
        if constexpr (!WAVE) {
            // a lane group per row; its valid partials' rows up to 8 at a time
            const char* po = static_cast<const char*>(a.po);
            for (uint32_t rl = group; rl < nr; rl += groups) {
                const uint32_t n = nv_lds[rl];
                const int64_t ooff = o_lds[rl];
                const bool have = ooff >= 0;
                char* orow = static_cast<char*>(a.out) + (have ? ooff : 0);
                const int64_t* offs = q_lds + rl * a.P;
                const float* wks = w_lds + rl * a.P;
                constexpr int VPL = kCombineNarrowVpl;
                for (uint32_t kb = 0; kb < a.cv; kb += G * VPL) {
                    bool kin[VPL];
                    uint32_t kbyte[VPL];
                    float acc[VPL][E];
#pragma unroll
                    for (int v = 0; v < VPL; ++v) {
                        const uint32_t idx = kb + gl + uint32_t(v) * G;
                        kin[v] = idx < a.cv;
                        kbyte[v] = (kin[v] ? idx : a.cv - 1) * uint32_t(W);
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            acc[v][e] = 0.0f;
                    }
                    constexpr uint32_t NB = kCombineNarrowBatch;
                    if constexpr (CAM_COMBINE_NARROW_PIPE) {
                        // two register sets take turns: partial kk + 1's payload
                        // is requested before partial kk is accumulated, so one
                        // request stays in flight while the other is consumed
                        typedef typename VecOf<W>::type V;
                        V xa[VPL], xb[VPL];
                        auto fetch = [&](V (&x)[VPL], uint32_t kk) {
                            const int64_t o1 = offs[kk];
#pragma unroll
                            for (int v = 0; v < VPL; ++v)
                                x[v] = ld_at<W, NTL>(po + o1 + kbyte[v]);
                        };
                        auto take = [&](const V (&x)[VPL], uint32_t kk) {
                            const float wv = wks[kk];
#pragma unroll
                            for (int v = 0; v < VPL; ++v) {
                                const Halves<W> xh = __builtin_bit_cast(Halves<W>, x[v]);
#pragma unroll
                                for (int e = 0; e < E; ++e)
                                    acc[v][e] = fmaf(wv, half_to_f32<FP16>(xh.h[e]), acc[v][e]);
                            }
                        };
                        if (n > 0) {
                            fetch(xa, 0);
                            uint32_t kk = 0;
                            for (; kk + 2 < n; kk += 2) {
                                fetch(xb, kk + 1);
                                issue_fence();
                                take(xa, kk);
                                issue_fence();
                                fetch(xa, kk + 2);
                                issue_fence();
                                take(xb, kk + 1);
                                issue_fence();
                            }
                            if (kk + 1 < n) {
                                fetch(xb, kk + 1);
                                take(xa, kk);
                                take(xb, kk + 1);
                            } else {
                                take(xa, kk);
                            }
                        }
                    } else
                    for (uint32_t k0 = 0; k0 < n; k0 += NB) {
                        const uint32_t cnt = n - k0 < NB ? n - k0 : NB;
                        const int64_t* o = offs + k0;
                        const float* wk = wks + k0;
                        switch (cnt) {
                        case 8: if constexpr (NB >= 8) combine_rows<8, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        case 7: if constexpr (NB >= 7) combine_rows<7, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        case 6: if constexpr (NB >= 6) combine_rows<6, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        case 5: if constexpr (NB >= 5) combine_rows<5, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        case 4: if constexpr (NB >= 4) combine_rows<4, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        case 3: if constexpr (NB >= 3) combine_rows<3, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        case 2: if constexpr (NB >= 2) combine_rows<2, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        default: combine_rows<1, W, FP16, NTL, VPL>(po, o, wk, kbyte, acc); break;
                        }
                    }
#pragma unroll
                    for (int v = 0; v < VPL; ++v)
                        if (have && kin[v])
                            st_at<W, NTS>(orow + kbyte[v], round_payload<W, FP16>(acc[v]));
                }
            }
            continue;
        }
        const uint32_t first = WAVE ? uniform32(group * RF) : group * RF;
        for (uint32_t rl0 = first; rl0 < nr; rl0 += groups * RF) {
            uint32_t rl[RF];
            bool have[RF];
            uint64_t msk[RF];
            char* orow[RF];
            const char* prow[RF];
#pragma unroll
            for (int f = 0; f < RF; ++f) {
                rl[f] = rl0 + f;
                have[f] = rl[f] < nr;
                if (!have[f])
                    rl[f] = rl0;  // stands in for the missing row; nothing is stored for it
                const uint64_t row = row0 + rl[f];
                const uint32_t t = fdiv(uint32_t(row), a.div_H);
                const uint32_t h = uint32_t(row) - t * a.H;
                msk[f] = WAVE ? uniform64(m_lds[rl[f]]) : m_lds[rl[f]];
                const int64_t ooff = WAVE ? int64_t(uniform64(uint64_t(o_lds[rl[f]]))) : o_lds[rl[f]];
                have[f] = have[f] && ooff >= 0;
                orow[f] = static_cast<char*>(a.out) + (ooff >= 0 ? ooff : 0);
                // a row without valid partials reads (and discards) its own output
                // row, so that no invalid partial row is ever read
                prow[f] = msk[f] ? static_cast<const char*>(a.po) + int64_t(t) * a.po_st_b + int64_t(h) * a.po_sh_b
                                 : orow[f];
            }
            for (uint32_t kb = 0; kb < a.cv; kb += G) {
                const bool kin = kb + gl < a.cv;
                const uint32_t k = kin ? kb + gl : a.cv - 1;
                float acc[RF][E];
                uint64_t m[RF];
#pragma unroll
                for (int f = 0; f < RF; ++f) {
                    m[f] = msk[f];
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        acc[f][e] = 0.0f;
                }
                for (;;) {
                    int idx[RF][CH];
                    float wv[RF][CH];
                    bool tk[RF][CH];
                    bool any = false;
#pragma unroll
                    for (int f = 0; f < RF; ++f) {
                        int last = msk[f] ? __builtin_ctzll(msk[f]) : 0;
#pragma unroll
                        for (int u = 0; u < CH; ++u) {
                            const bool take = m[f] != 0;
                            const int p = take ? __builtin_ctzll(m[f]) : last;
                            m[f] = take ? (m[f] & (m[f] - 1)) : m[f];
                            idx[f][u] = p;
                            last = p;
                            tk[f][u] = take;
                            const float wl = w_lds[rl[f] * a.P + uint32_t(p)];
                            wv[f][u] = WAVE ? __uint_as_float(uniform32(__float_as_uint(wl))) : wl;
                        }
                        any = any || m[f] != 0;
                    }
                    V x[RF][CH];
#pragma unroll
                    for (int f = 0; f < RF; ++f)
#pragma unroll
                        for (int u = 0; u < CH; ++u)
                            x[f][u] = ld_at<W, NTL>(prow[f] + int64_t(k) * W + int64_t(idx[f][u]) * a.po_sp_b);
                    issue_fence();
#pragma unroll
                    for (int f = 0; f < RF; ++f)
#pragma unroll
                        for (int u = 0; u < CH; ++u) {
                            const Halves<W> xh = __builtin_bit_cast(Halves<W>, x[f][u]);
#pragma unroll
                            for (int e = 0; e < E; ++e) {
                                const float v = fmaf(wv[f][u], half_to_f32<FP16>(xh.h[e]), acc[f][e]);
                                acc[f][e] = tk[f][u] ? v : acc[f][e];
                            }
                        }
                    if (!any)
                        break;
                }
#pragma unroll
                for (int f = 0; f < RF; ++f) {
                    if (have[f] && kin) {
                        Halves<W> oh;
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            oh.h[e] = f32_to_half<FP16>(msk[f] ? acc[f][e] : 0.0f);
                        st_at<W, NTS>(orow[f] + int64_t(k) * W, __builtin_bit_cast(V, oh));
                    }
                }
            }
        }
    }
}

// Rows of at least 64 vectors, without LDS or barriers: every wave owns a
// stream of rows (row = wave, wave + n_waves, ...).  A row's P statistics sit
// in lanes 0..P-1 and are reduced across the wave; each valid partial's weight
// is read into a scalar register; the next row's LSEs are loaded while the
// current row's payload streams, so a row costs one memory round trip.
__device__ __forceinline__ float wave_max(float v)
{
    for (int off = 32; off > 0; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
    for (int off = 32; off > 0; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// The next N valid partials of a row whose statistics sit in the wave's lanes:
// their indices come off the wave-uniform mask m (lowest first), their
// normalised weights are read from the owning lanes, then all N payload
// vectors are loaded before any is accumulated.
template <int N, int W, bool FP16, bool NTL>
__device__ __forceinline__ void stream_rows(const char* prow, int64_t sp_b, uint32_t kbyte, uint64_t& m, float wn,
                                            float (&acc)[W / 2])
{
    typedef typename VecOf<W>::type V;
    constexpr int E = W / 2;
    int idx[N];
    float w[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
        idx[u] = __builtin_ctzll(m);
        m &= m - 1;
        w[u] = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(wn)), idx[u])));
    }
    V x[N];
#pragma unroll
    for (int u = 0; u < N; ++u)
        x[u] = ld_at<W, NTL>(prow + kbyte + int64_t(idx[u]) * sp_b);
    issue_fence();
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const Halves<W> xh = __builtin_bit_cast(Halves<W>, x[u]);
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] = fmaf(w[u], half_to_f32<FP16>(xh.h[e]), acc[e]);
    }
}

template <int CZ, typename Rec>
__device__ __forceinline__ float row_stat(const Rec& a, uint64_t row, uint32_t lane)
{
    if (row >= a.n_rows)  // wave-uniform
        return -__builtin_inff();
    const uint32_t t = fdiv(uint32_t(row), a.div_H);
    const uint32_t h = uint32_t(row) - t * a.H;
    if (CZ != kAll) {
        const int32_t seq = wave_seq_of_token(a.cu, a.nseq, t);  // one token per wave: the wave searches
        if (lane >= a.P || !admitted_partial<CZ>(a, a.cu, seq, lane, t))
            return -__builtin_inff();
    } else if (lane >= a.P) {
        return -__builtin_inff();
    }
    return a.pl[int64_t(lane) * a.pl_sp + int64_t(t) * a.pl_st + int64_t(h) * a.pl_sh];
}

template <int W, bool FP16, int CZ, int OM>
__global__ __launch_bounds__(kThreads) void k_combine_stream(Combine a)
{
    constexpr int E = W / 2;
    constexpr int CH = kCombineBatchWave;
    constexpr bool NTL = (CAM_NT_COMBINE & 1) != 0, NTS = (CAM_NT_COMBINE & 2) != 0;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wpb = blockDim.x >> 6;
    const uint64_t blk = a.xcd ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint64_t n_waves = uint64_t(gridDim.x) * wpb;
    uint64_t row = blk * wpb + uniform32(threadIdx.x >> 6);
    float L_next = row_stat<CZ>(a, row, lane);
    for (; row < a.n_rows; row += n_waves) {
        const float L = L_next;
        L_next = row_stat<CZ>(a, row + n_waves, lane);  // in flight during this row
        const uint32_t t = fdiv(uint32_t(row), a.div_H);
        const uint32_t h = uint32_t(row) - t * a.H;
        const bool valid = __builtin_isfinite(L);
        const float M = wave_max(valid ? L : -__builtin_inff());
        const float w = valid ? weight_exp(L - M) : 0.0f;
        const float Z = wave_sum(w);
        const uint64_t vmask = __ballot(valid);
        const float wn = w * (vmask ? recip(Z) : 0.0f);
        int64_t o_off, l_off;
        if (OM == 0) {
            o_off = int64_t(t) * a.o_st_b + int64_t(h) * a.o_sh_b;
            l_off = int64_t(t) * a.lo_st + int64_t(h) * a.lo_sh;
        } else {
            int64_t g;
            if (OM == 1) {
                const uint32_t tq = fdiv(h, a.div_Hp);
                g = int64_t(tq) * a.Hq + int64_t(t) * a.Hp + (h - tq * a.Hp);
            } else {
                g = varlen_token_row(a.cu, a, wave_seq_of_token(a.cu, a.nseq, t), t) * a.H + h;
            }
            const bool in = g >= 0 && uint64_t(g) < a.n_rows;
            o_off = in ? g * int64_t(a.o_row_b) : -1;
            l_off = in ? g : -1;
        }
        if (lane == 0 && a.lse_out && l_off >= 0)
            a.lse_out[l_off] = vmask ? M + logf(Z) : -__builtin_inff();
        const bool have = o_off >= 0;
        char* orow = static_cast<char*>(a.out) + (have ? o_off : 0);
        const char* prow = vmask ? static_cast<const char*>(a.po) + int64_t(t) * a.po_st_b + int64_t(h) * a.po_sh_b
                                 : orow;
        const uint32_t n = uint32_t(__builtin_popcountll(vmask));
        for (uint32_t kb = 0; kb < a.cv; kb += 64) {
            const bool kin = kb + lane < a.cv;
            const uint32_t kbyte = (kin ? kb + lane : a.cv - 1) * uint32_t(W);
            float acc[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[e] = 0.0f;
            uint64_t m = vmask;  // wave-uniform: the valid partials not yet taken
            for (uint32_t k0 = 0; k0 < n; k0 += CH) {
                const uint32_t cnt = n - k0 < uint32_t(CH) ? n - k0 : uint32_t(CH);
                switch (cnt) {
                case 8: if constexpr (CH >= 8) stream_rows<8, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                case 7: if constexpr (CH >= 7) stream_rows<7, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                case 6: if constexpr (CH >= 6) stream_rows<6, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                case 5: if constexpr (CH >= 5) stream_rows<5, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                case 4: if constexpr (CH >= 4) stream_rows<4, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                case 3: if constexpr (CH >= 3) stream_rows<3, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                case 2: if constexpr (CH >= 2) stream_rows<2, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                default: stream_rows<1, W, FP16, NTL>(prow, a.po_sp_b, kbyte, m, wn, acc); break;
                }
            }
            if (have && kin)
                st_at<W, NTS>(orow + kbyte, round_payload<W, FP16>(acc));
        }
    }
}

// ---------------------------------------------------------------------------
// Online two-way merge (ring / context-parallel accumulation)
// ---------------------------------------------------------------------------

// Per row: La = accumulator LSE (-inf: empty), Lb = partial LSE; the valid ones
// (finite) are combined with weights exp(L - max); the accumulator row is
// rewritten in fp32 and, if asked, the rounded payload too.  A group of G lanes
// covers a row, 4 elements per lane; an empty accumulator row is not read, and
// an invalid partial's row is never read (its lane re-reads the accumulator
// row, a valid address, and discards it).
template <bool FP16, bool FINAL>
__global__ __launch_bounds__(kThreads) void k_merge(Merge a)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const uint32_t G = 1u << a.g_log2;
    const uint32_t gl = threadIdx.x & (G - 1u);
    const uint64_t rows_per_block = uint64_t(kThreads) >> a.g_log2;
    const uint64_t blk = CAM_XCD_MERGE ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    for (uint64_t rb = blk * rows_per_block; rb < a.n_rows; rb += uint64_t(gridDim.x) * rows_per_block) {
        const uint64_t row = rb + (threadIdx.x >> a.g_log2);
        if (row >= a.n_rows)
            continue;
        const uint32_t t = fdiv(uint32_t(row), a.div_H);
        const uint32_t h = uint32_t(row) - t * a.H;
        const float La = a.acc_lse[int64_t(t) * a.al_st + int64_t(h) * a.al_sh];
        const float Lb = a.part_lse[int64_t(t) * a.pl_st + int64_t(h) * a.pl_sh];
        const bool va = __builtin_isfinite(La), vb = __builtin_isfinite(Lb);
        const float M = va ? (vb ? fmaxf(La, Lb) : La) : Lb;
        const float wa = va ? expf(La - M) : 0.0f;
        const float wb = vb ? expf(Lb - M) : 0.0f;
        const float Z = wa + wb;
        const bool any = va || vb;
        const float sa = any ? wa / Z : 0.0f, sb = any ? wb / Z : 0.0f;
        float* arow = a.acc + int64_t(t) * a.a_st + int64_t(h) * a.a_sh;
        const char* prow = vb ? static_cast<const char*>(a.part) + int64_t(t) * a.p_st_b + int64_t(h) * a.p_sh_b
                              : reinterpret_cast<const char*>(arow);
        char* frow = FINAL ? static_cast<char*>(a.fin) + int64_t(t) * a.f_st_b + int64_t(h) * a.f_sh_b : nullptr;
        for (uint32_t k = gl; k < a.cv; k += G) {
            // an empty accumulator (the first hop) is not read
            constexpr bool NTL = (CAM_NT_MERGE & 1) != 0, NTS = (CAM_NT_MERGE & 2) != 0;
            f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
            const f32x4* xa = reinterpret_cast<const f32x4*>(arow + 4 * k);
            const u32x2* yp = reinterpret_cast<const u32x2*>(prow + 8 * k);
            if (va)
                x = NTL ? __builtin_nontemporal_load(xa) : *xa;
            const u32x2 y = NTL ? __builtin_nontemporal_load(yp) : *yp;
            issue_fence();
            const float b0 = FP16 ? fp16_lo(y.x) : bf16_lo(y.x), b1 = FP16 ? fp16_hi(y.x) : bf16_hi(y.x);
            const float b2 = FP16 ? fp16_lo(y.y) : bf16_lo(y.y), b3 = FP16 ? fp16_hi(y.y) : bf16_hi(y.y);
            f32x4 r;
            r.x = (va ? sa * x.x : 0.0f) + (vb ? sb * b0 : 0.0f);
            r.y = (va ? sa * x.y : 0.0f) + (vb ? sb * b1 : 0.0f);
            r.z = (va ? sa * x.z : 0.0f) + (vb ? sb * b2 : 0.0f);
            r.w = (va ? sa * x.w : 0.0f) + (vb ? sb * b3 : 0.0f);
            if (NTS)
                __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(arow + 4 * k));
            else
                *reinterpret_cast<f32x4*>(arow + 4 * k) = r;
            if (FINAL) {
                u32x2 o;
                if (FP16) {
                    o.x = f32_to_fp16_bits(r.x) | (f32_to_fp16_bits(r.y) << 16);
                    o.y = f32_to_fp16_bits(r.z) | (f32_to_fp16_bits(r.w) << 16);
                } else {
                    o.x = f32_to_bf16_bits(r.x) | (f32_to_bf16_bits(r.y) << 16);
                    o.y = f32_to_bf16_bits(r.z) | (f32_to_bf16_bits(r.w) << 16);
                }
                if (NTS)
                    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(frow + 8 * k));
                else
                    *reinterpret_cast<u32x2*>(frow + 8 * k) = o;
            }
        }
        if (gl == 0)
            a.acc_lse[int64_t(t) * a.al_st + int64_t(h) * a.al_sh] = any ? M + logf(Z) : -__builtin_inff();
    }
}

cam_status launch_merge(const Merge& a, void* stream)
{
    const void* fn = a.fin ? (a.fp16 ? reinterpret_cast<const void*>(&k_merge<true, true>)
                                     : reinterpret_cast<const void*>(&k_merge<false, true>))
                           : (a.fp16 ? reinterpret_cast<const void*>(&k_merge<true, false>)
                                     : reinterpret_cast<const void*>(&k_merge<false, false>));
    const uint64_t rows_per_block = uint64_t(kThreads) >> a.g_log2;
    return launch(fn, a, (a.n_rows + rows_per_block - 1) / rows_per_block, stream, "lse_merge");
}

// ---------------------------------------------------------------------------
// Gradient of the combine
// ---------------------------------------------------------------------------

// Tiles of RB rows, three phases.  Phase 1 recomputes each row's normalised
// weights exactly as the forward does (same admission, max and sum), with the
// statistics lanes of the forward.  Phase 2 streams each row once: the
// upstream gradient g, then the valid partials' O rows in branch-free batches;
// the lanes of a row form <g, O_p> (a shuffle reduction across the row's lanes,
// summed over the row's vector blocks in LDS) and write dO_p = w_p g for every
// partial, zero for those outside the valid set.  Phase 3 forms
// dL_p = w_p (<g, O_p> - sum_q w_q <g, O_q> + g_lse) on the statistics lanes.
// As in the forward, an invalid or masked partial's O row is never read.
// Dot product of two payload vectors in fp32: pairs of bf16/fp16 elements
// through the packed dot instruction (products exact, fp32 accumulation),
// single elements through fma.
template <int W, bool FP16>
__device__ __forceinline__ float payload_dot(typename VecOf<W>::type a, typename VecOf<W>::type b, float d)
{
    constexpr int E = W / 2;
    if constexpr (E % 2 == 0) {
        struct Words {
            uint32_t w[E / 2];
        };
        const Words aw = __builtin_bit_cast(Words, a), bw = __builtin_bit_cast(Words, b);
#pragma unroll
        for (int i = 0; i < E / 2; ++i) {
            if constexpr (FP16) {
                typedef _Float16 h2 __attribute__((ext_vector_type(2)));
                d = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, aw.w[i]), __builtin_bit_cast(h2, bw.w[i]), d, false);
            } else {
                typedef __bf16 b2 __attribute__((ext_vector_type(2)));
                d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, aw.w[i]), __builtin_bit_cast(b2, bw.w[i]), d,
                                                    false);
            }
        }
        return d;
    } else {
        const Halves<W> ah = __builtin_bit_cast(Halves<W>, a), bh = __builtin_bit_cast(Halves<W>, b);
#pragma unroll
        for (int e = 0; e < E; ++e)
            d = fmaf(half_to_f32<FP16>(ah.h[e]), half_to_f32<FP16>(bh.h[e]), d);
        return d;
    }
}

// Gradient, compacted form: the next N valid partials of a row, <g, O_p> of
// this lane's vectors added to the lane's slot of each partial in LDS (a
// clamped tail vector contributes nothing).
template <int N, int W, bool FP16, bool NTL, int VPL>
__device__ __forceinline__ void bwd_dots(const char* po, const int64_t* offs, const uint32_t (&kbyte)[VPL],
                                         const bool (&kin)[VPL], const typename VecOf<W>::type (&gv)[VPL],
                                         float* dd, uint32_t G)
{
    typedef typename VecOf<W>::type V;
    int64_t o[N];
#pragma unroll
    for (int u = 0; u < N; ++u)
        o[u] = offs[u];
    V x[N][VPL];
#pragma unroll
    for (int u = 0; u < N; ++u)
#pragma unroll
        for (int v = 0; v < VPL; ++v)
            x[u][v] = ld_at<W, NTL>(po + o[u] + kbyte[v]);
    issue_fence();
#pragma unroll
    for (int u = 0; u < N; ++u) {
        float d = 0.0f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
            const float dv = payload_dot<W, FP16>(x[u][v], gv[v], 0.0f);
            d += kin[v] ? dv : 0.0f;
        }
        dd[u * G] += d;
    }
}

// COMPACT: each row's valid partials as a compacted list (byte offsets) in
// LDS, loaded with exact counts; every lane adds its share of <g, O_p> to its
// own slot of a per-(row, valid partial) table, reduced in phase 3 (no
// cross-lane shuffles in the payload loop); the workgroup holds one lane
// group per row.  Otherwise a lane group reduces each dot product with
// shuffles and accumulates it per partial.
template <int W, bool FP16, int CZ, bool COMPACT>
__global__ __launch_bounds__(kThreads) void k_combine_bwd(CombineBwd a)
{
    typedef typename VecOf<W>::type V;
    constexpr int E = W / 2;
    constexpr int CH = kCombineBwdBatch;
    constexpr bool NTL = (CAM_NT_COMBINE_BWD & 1) != 0, NTS = (CAM_NT_COMBINE_BWD & 2) != 0;
    extern __shared__ float smem[];
    const uint32_t RB = a.rows_per_tile;
    const uint32_t G = 1u << a.g_log2;
    // COMPACT: offsets [RB*P] int64, masks [RB], weights [RB*P], per-lane dot
    // products [RB*P*G], g_lse [RB], counts [RB], cu
    int64_t* q_lds = reinterpret_cast<int64_t*>(smem);
    uint64_t* mc_lds = reinterpret_cast<uint64_t*>(q_lds + RB * a.P);
    float* wc_lds = reinterpret_cast<float*>(mc_lds + RB);
    float* dd_lds = wc_lds + RB * a.P;
    float* glc_lds = dd_lds + RB * a.P * G;
    uint32_t* nv_lds = reinterpret_cast<uint32_t*>(glc_lds + RB);
    // otherwise: weights [RB*P], <g, O_p> [RB*P], g_lse [RB], masks [RB], cu
    float* w_lds = COMPACT ? wc_lds : smem;                                    // RB * P weights
    float* d_lds = w_lds + RB * a.P;                                           // RB * P  <g, O_p>
    float* gl_lds = COMPACT ? glc_lds : d_lds + RB * a.P;                      // RB  g_lse
    uint64_t* m_lds = COMPACT ? mc_lds : reinterpret_cast<uint64_t*>(gl_lds + ((RB + 1) & ~1u));  // RB masks
    int32_t* cu_lds = COMPACT ? reinterpret_cast<int32_t*>(nv_lds + RB)
                              : reinterpret_cast<int32_t*>(m_lds + RB);        // nseq + 1 (varlen)
    const bool cached = CZ != kAll && a.nseq < kCuCache;
    if (cached)
        for (uint32_t i = threadIdx.x; i <= uint32_t(a.nseq); i += kThreads)
            cu_lds[i] = a.cu[i];

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t GP = 1u << a.gp_log2;
    const uint32_t sp = lane & (GP - 1u);
    const uint32_t sbase = lane & ~(GP - 1u);
    const uint64_t spmask = GP == 64u ? ~0ull : ((1ull << GP) - 1ull);
    const uint32_t gl = lane & (G - 1u);
    const uint32_t nthr = blockDim.x;
    const uint32_t groups = nthr >> a.g_log2;
    const uint32_t group = threadIdx.x >> a.g_log2;

    for (uint64_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
        const uint64_t row0 = tile * RB;
        // ---- phase 1: weights of the tile's rows
        __syncthreads();
        if (COMPACT)
            for (uint32_t i = threadIdx.x; i < RB * a.P * G; i += nthr)
                dd_lds[i] = 0.0f;
        for (uint32_t base = 0; base < RB * GP; base += nthr) {
            const uint32_t tau = base + threadIdx.x;
            const uint32_t rl = tau >> a.gp_log2;
            const uint64_t row = row0 + rl;
            const bool live = rl < RB && row < a.n_rows;
            uint32_t t = 0, h = 0;
            if (live) {
                t = fdiv(uint32_t(row), a.div_H);
                h = uint32_t(row) - t * a.H;
            }
            int32_t seq = 0;  // the token's sequence (the causal rules)
            if (CZ != kAll) {
                const uint32_t wl = (base + (threadIdx.x & ~63u)) >> a.gp_log2;  // the wave's first row
                seq = tile_token_seq(a, cu_lds, cached, wl < RB && row0 + wl < a.n_rows, row0 + wl, live, t);
            }
            bool valid = false;
            float L = -__builtin_inff();
            if (live && sp < a.P) {
                bool admitted = true;
                if (CZ != kAll)
                    admitted = cached ? admitted_partial<CZ>(a, cu_lds, seq, sp, t)
                                      : admitted_partial<CZ>(a, a.cu, seq, sp, t);
                if (admitted) {
                    L = a.pl[int64_t(sp) * a.pl_sp + int64_t(t) * a.pl_st + int64_t(h) * a.pl_sh];
                    valid = __builtin_isfinite(L);
                }
            }
            float M = valid ? L : -__builtin_inff();
            for (uint32_t off = GP >> 1; off > 0; off >>= 1)
                M = fmaxf(M, __shfl_xor(M, int(off), int(GP)));
            const uint64_t vmask = (__ballot(valid) >> sbase) & spmask;
            const float w = valid ? expf(L - M) : 0.0f;
            float Z = w;
            for (uint32_t off = GP >> 1; off > 0; off >>= 1)
                Z += __shfl_xor(Z, int(off), int(GP));
            if (live) {
                const float iz = vmask ? 1.0f / Z : 0.0f;
                if (sp < a.P) {
                    w_lds[rl * a.P + sp] = w * iz;
                    if (!COMPACT)
                        d_lds[rl * a.P + sp] = 0.0f;
                }
                if (COMPACT && valid) {
                    const uint32_t slot = uint32_t(__builtin_popcountll(vmask & ((1ull << sp) - 1ull)));
                    q_lds[rl * a.P + slot] =
                        int64_t(sp) * a.po_sp_b + int64_t(t) * a.po_st_b + int64_t(h) * a.po_sh_b;
                }
                if (sp == 0) {
                    m_lds[rl] = vmask;
                    gl_lds[rl] = a.gl ? a.gl[int64_t(t) * a.gl_st + int64_t(h) * a.gl_sh] : 0.0f;
                    if (COMPACT)
                        nv_lds[rl] = uint32_t(__builtin_popcountll(vmask));
                }
            }
        }
        __syncthreads();

        // ---- phase 2: one pass over each row's payload
        const uint64_t left = a.n_rows - row0;
        const uint32_t nr = left < RB ? uint32_t(left) : RB;
        if constexpr (COMPACT) {
            constexpr int VPL = kCombineBwdVpl;
            constexpr uint32_t NB = kCombineBwdNarrowBatch;
            const char* po = static_cast<const char*>(a.po);
            for (uint32_t rl = group; rl < nr; rl += groups) {
                const uint64_t row = row0 + rl;
                const uint32_t t = fdiv(uint32_t(row), a.div_H);
                const uint32_t h = uint32_t(row) - t * a.H;
                const uint64_t msk = m_lds[rl];
                const uint32_t n = nv_lds[rl];
                const char* grow = static_cast<const char*>(a.go) + int64_t(t) * a.go_st_b + int64_t(h) * a.go_sh_b;
                char* drow = static_cast<char*>(a.dpo) + int64_t(t) * a.dpo_st_b + int64_t(h) * a.dpo_sh_b;
                const int64_t* offs = q_lds + rl * a.P;
                float* ddr = dd_lds + rl * a.P * G + gl;
                for (uint32_t kb = 0; kb < a.cv; kb += G * VPL) {
                    bool kin[VPL];
                    uint32_t kbyte[VPL];
                    V gv[VPL];
#pragma unroll
                    for (int v = 0; v < VPL; ++v) {
                        const uint32_t idx = kb + gl + uint32_t(v) * G;
                        kin[v] = idx < a.cv;
                        kbyte[v] = (kin[v] ? idx : a.cv - 1) * uint32_t(W);
                        gv[v] = V{};
                    }
                    if (n) {  // the upstream gradient is read only where some partial is valid
#pragma unroll
                        for (int v = 0; v < VPL; ++v)
                            gv[v] = ld_at<W, NTL>(grow + kbyte[v]);
                    }
                    for (uint32_t k0 = 0; k0 < n; k0 += NB) {
                        const uint32_t cnt = n - k0 < NB ? n - k0 : NB;
                        const int64_t* o = offs + k0;
                        float* dd = ddr + k0 * G;
                        switch (cnt) {
                        case 8: if constexpr (NB >= 8) bwd_dots<8, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        case 7: if constexpr (NB >= 7) bwd_dots<7, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        case 6: if constexpr (NB >= 6) bwd_dots<6, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        case 5: if constexpr (NB >= 5) bwd_dots<5, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        case 4: if constexpr (NB >= 4) bwd_dots<4, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        case 3: if constexpr (NB >= 3) bwd_dots<3, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        case 2: if constexpr (NB >= 2) bwd_dots<2, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        default: bwd_dots<1, W, FP16, NTL, VPL>(po, o, kbyte, kin, gv, dd, G); break;
                        }
                    }
                    // dO_p = w_p g for every partial (exact zero outside the valid set)
                    float gf[VPL][E];
#pragma unroll
                    for (int v = 0; v < VPL; ++v) {
                        const Halves<W> gh = __builtin_bit_cast(Halves<W>, gv[v]);
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            gf[v][e] = half_to_f32<FP16>(gh.h[e]);
                    }
                    for (uint32_t p = 0; p < a.P; ++p) {
                        const bool vp = ((msk >> p) & 1ull) != 0;
                        const float wp = w_lds[rl * a.P + p];
#pragma unroll
                        for (int v = 0; v < VPL; ++v) {
                            float y[E];
#pragma unroll
                            for (int e = 0; e < E; ++e)
                                y[e] = wp * gf[v][e];
                            const V out = vp ? round_payload<W, FP16>(y) : V{};
                            if (kin[v])
                                st_at<W, NTS>(drow + int64_t(kbyte[v]) + int64_t(p) * a.dpo_sp_b, out);
                        }
                    }
                }
            }
        } else
        for (uint32_t rl = group; rl < nr; rl += groups) {
            const uint64_t row = row0 + rl;
            const uint32_t t = fdiv(uint32_t(row), a.div_H);
            const uint32_t h = uint32_t(row) - t * a.H;
            const uint64_t msk = m_lds[rl];
            const char* prow = static_cast<const char*>(a.po) + int64_t(t) * a.po_st_b + int64_t(h) * a.po_sh_b;
            const char* grow = static_cast<const char*>(a.go) + int64_t(t) * a.go_st_b + int64_t(h) * a.go_sh_b;
            char* drow = static_cast<char*>(a.dpo) + int64_t(t) * a.dpo_st_b + int64_t(h) * a.dpo_sh_b;
            for (uint32_t kb = 0; kb < a.cv; kb += G) {
                const bool kin = kb + gl < a.cv;
                const uint32_t k = kin ? kb + gl : a.cv - 1;
                float ge[E];
                if (msk) {
                    const Halves<W> gh = __builtin_bit_cast(Halves<W>, ld_at<W, NTL>(grow + int64_t(k) * W));
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        ge[e] = half_to_f32<FP16>(gh.h[e]);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        ge[e] = 0.0f;
                }
                // <g, O_p> over the valid partials, CH rows per batch; a short
                // batch repeats its last valid partial and discards the result
                uint64_t m = msk;
                int last = msk ? __builtin_ctzll(msk) : 0;
                while (m) {
                    int idx[CH];
                    bool tk[CH];
#pragma unroll
                    for (int u = 0; u < CH; ++u) {
                        const bool take = m != 0;
                        const int p = take ? __builtin_ctzll(m) : last;
                        m = take ? (m & (m - 1)) : m;
                        idx[u] = p;
                        last = p;
                        tk[u] = take;
                    }
                    V x[CH];
#pragma unroll
                    for (int u = 0; u < CH; ++u)
                        x[u] = ld_at<W, NTL>(prow + int64_t(k) * W + int64_t(idx[u]) * a.po_sp_b);
                    issue_fence();
#pragma unroll
                    for (int u = 0; u < CH; ++u) {
                        const Halves<W> xh = __builtin_bit_cast(Halves<W>, x[u]);
                        float d = 0.0f;
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            d = fmaf(ge[e], half_to_f32<FP16>(xh.h[e]), d);
                        d = kin ? d : 0.0f;  // a clamped tail lane repeats a vector
                        for (uint32_t off = G >> 1; off > 0; off >>= 1)
                            d += __shfl_xor(d, int(off), int(G));
                        if (gl == 0 && tk[u])
                            d_lds[rl * a.P + uint32_t(idx[u])] += d;
                    }
                }
                // dO_p = w_p g for every partial (exact zero outside the valid set)
                if (kin)
                    for (uint32_t p = 0; p < a.P; ++p) {
                        const float wp = w_lds[rl * a.P + p];
                        const bool vp = ((msk >> p) & 1ull) != 0;
                        Halves<W> oh;
#pragma unroll
                        for (int e = 0; e < E; ++e)
                            oh.h[e] = f32_to_half<FP16>(vp ? wp * ge[e] : 0.0f);
                        st_at<W, NTS>(drow + int64_t(k) * W + int64_t(p) * a.dpo_sp_b, __builtin_bit_cast(V, oh));
                    }
            }
        }
        __syncthreads();

        // ---- phase 3: gradient of the partial LSEs
        for (uint32_t base = 0; base < RB * GP; base += nthr) {
            const uint32_t tau = base + threadIdx.x;
            const uint32_t rl = tau >> a.gp_log2;
            const uint64_t row = row0 + rl;
            const bool live = rl < RB && row < a.n_rows;
            const bool mine = live && sp < a.P;
            const float w = mine ? w_lds[rl * a.P + sp] : 0.0f;
            float d = 0.0f;
            if (COMPACT) {
                const uint64_t vm = mine ? m_lds[rl] : 0ull;
                if (((vm >> sp) & 1ull) != 0) {
                    const uint32_t slot = uint32_t(__builtin_popcountll(vm & ((1ull << sp) - 1ull)));
                    const float* q = dd_lds + (rl * a.P + slot) * G;
                    for (uint32_t j = 0; j < G; ++j)
                        d += q[j];
                }
            } else {
                d = mine ? d_lds[rl * a.P + sp] : 0.0f;
            }
            float s = w * d;
            for (uint32_t off = GP >> 1; off > 0; off >>= 1)
                s += __shfl_xor(s, int(off), int(GP));
            if (mine) {
                const uint32_t t = fdiv(uint32_t(row), a.div_H);
                const uint32_t h = uint32_t(row) - t * a.H;
                const bool valid = ((m_lds[rl] >> sp) & 1ull) != 0;
                a.dpl[int64_t(sp) * a.dpl_sp + int64_t(t) * a.dpl_st + int64_t(h) * a.dpl_sh] =
                    valid ? w * (d - s + gl_lds[rl]) : 0.0f;
            }
        }
    }
}

// Gradient for rows of at least 64 vectors, without LDS or barriers (the
// forward's row-stream layout): one wave per row.  The row's P statistics sit
// in lanes 0..P-1 and give the forward's normalised weights; the upstream
// gradient g is read once; each valid partial's <g, O_p> is formed per lane
// with the packed dot instruction and summed across the wave into lane p;
// every partial's dO_p = w_p g is written (exact zero outside the valid set);
// lane p then writes dL_p = w_p (<g, O_p> - sum_q w_q <g, O_q> + g_lse).
template <int N, int W, bool FP16, bool NTL>
__device__ __forceinline__ void stream_dots(const char* prow, int64_t sp_b, uint32_t kbyte, bool kin, uint64_t& m,
                                            typename VecOf<W>::type gv, uint32_t lane, float& dsum)
{
    typedef typename VecOf<W>::type V;
    int idx[N];
#pragma unroll
    for (int u = 0; u < N; ++u) {
        idx[u] = __builtin_ctzll(m);
        m &= m - 1;
    }
    V x[N];
#pragma unroll
    for (int u = 0; u < N; ++u)
        x[u] = ld_at<W, NTL>(prow + kbyte + int64_t(idx[u]) * sp_b);
    issue_fence();
#pragma unroll
    for (int u = 0; u < N; ++u) {
        const float d = wave_sum(kin ? payload_dot<W, FP16>(gv, x[u], 0.0f) : 0.0f);  // a clamped tail lane adds 0
        dsum += lane == uint32_t(idx[u]) ? d : 0.0f;
    }
}

template <int W, bool FP16, int CZ>
__global__ __launch_bounds__(kThreads) void k_combine_bwd_stream(CombineBwd a)
{
    typedef typename VecOf<W>::type V;
    constexpr int E = W / 2;
    constexpr int CH = kCombineBatchWave;
    constexpr bool NTL = (CAM_NT_COMBINE_BWD_STREAM & 1) != 0, NTS = (CAM_NT_COMBINE_BWD_STREAM & 2) != 0;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wpb = blockDim.x >> 6;
    const uint64_t blk = CAM_XCD_COMBINE_BWD_STREAM ? xcd_first(blockIdx.x, gridDim.x) : blockIdx.x;
    const uint64_t n_waves = uint64_t(gridDim.x) * wpb;
    uint64_t row = blk * wpb + uniform32(threadIdx.x >> 6);
    float L_next = row_stat<CZ>(a, row, lane);
    for (; row < a.n_rows; row += n_waves) {
        const float L = L_next;
        L_next = row_stat<CZ>(a, row + n_waves, lane);  // in flight during this row
        const uint32_t t = fdiv(uint32_t(row), a.div_H);
        const uint32_t h = uint32_t(row) - t * a.H;
        const bool valid = __builtin_isfinite(L);
        const float M = wave_max(valid ? L : -__builtin_inff());
        const float w = valid ? expf(L - M) : 0.0f;
        const float Z = wave_sum(w);
        const uint64_t vmask = __ballot(valid);
        const float wn = w * (vmask ? 1.0f / Z : 0.0f);
        const uint32_t n = uint32_t(__builtin_popcountll(vmask));
        const float glv = a.gl ? a.gl[int64_t(t) * a.gl_st + int64_t(h) * a.gl_sh] : 0.0f;
        const char* prow = static_cast<const char*>(a.po) + int64_t(t) * a.po_st_b + int64_t(h) * a.po_sh_b;
        const char* grow = static_cast<const char*>(a.go) + int64_t(t) * a.go_st_b + int64_t(h) * a.go_sh_b;
        char* drow = static_cast<char*>(a.dpo) + int64_t(t) * a.dpo_st_b + int64_t(h) * a.dpo_sh_b;
        float dsum = 0.0f;  // lane p: <g, O_p>
        for (uint32_t kb = 0; kb < a.cv; kb += 64) {
            const bool kin = kb + lane < a.cv;
            const uint32_t kbyte = (kin ? kb + lane : a.cv - 1) * uint32_t(W);
            // the upstream gradient is read only where some partial is valid
            const V gv = n ? ld_at<W, NTL>(grow + kbyte) : V{};
            uint64_t m = vmask;  // wave-uniform: the valid partials not yet taken
            for (uint32_t k0 = 0; k0 < n; k0 += CH) {
                const uint32_t cnt = n - k0 < uint32_t(CH) ? n - k0 : uint32_t(CH);
                switch (cnt) {
                case 8: if constexpr (CH >= 8) stream_dots<8, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                case 7: if constexpr (CH >= 7) stream_dots<7, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                case 6: if constexpr (CH >= 6) stream_dots<6, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                case 5: if constexpr (CH >= 5) stream_dots<5, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                case 4: if constexpr (CH >= 4) stream_dots<4, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                case 3: if constexpr (CH >= 3) stream_dots<3, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                case 2: if constexpr (CH >= 2) stream_dots<2, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                default: stream_dots<1, W, FP16, NTL>(prow, a.po_sp_b, kbyte, kin, m, gv, lane, dsum); break;
                }
            }
            // dO_p = w_p g for every partial (exact zero outside the valid set)
            float gf[E];
            const Halves<W> gh = __builtin_bit_cast(Halves<W>, gv);
#pragma unroll
            for (int e = 0; e < E; ++e)
                gf[e] = half_to_f32<FP16>(gh.h[e]);
            for (uint32_t p = 0; p < a.P; ++p) {
                const float wp = __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(wn)), int(p))));
                const bool vp = ((vmask >> p) & 1ull) != 0;
                float y[E];
#pragma unroll
                for (int e = 0; e < E; ++e)
                    y[e] = wp * gf[e];
                const V out = vp ? round_payload<W, FP16>(y) : V{};
                if (kin)
                    st_at<W, NTS>(drow + kbyte + int64_t(p) * a.dpo_sp_b, out);
            }
        }
        const float sw = wave_sum(wn * dsum);  // sum_q w_q <g, O_q>
        if (lane < a.P)
            a.dpl[int64_t(lane) * a.dpl_sp + int64_t(t) * a.dpl_st + int64_t(h) * a.dpl_sh] =
                valid ? wn * (dsum - sw + glv) : 0.0f;
    }
}

template <typename K>
const void* fn_ptr(K* k)
{
    return reinterpret_cast<const void*>(k);
}

// The admission rule of a launch record: none, the piece rule, or a plan's.
template <typename Rec>
int causal_rule(const Rec& a)
{
    return !a.cu ? kAll : a.first ? kPlan : kPieces;
}

template <int W, bool FP16, bool COMPACT>
const void* pick_combine_bwd(int cz)
{
    return cz == kPlan ? fn_ptr(&k_combine_bwd<W, FP16, kPlan, COMPACT>)
           : cz == kPieces ? fn_ptr(&k_combine_bwd<W, FP16, kPieces, COMPACT>)
                           : fn_ptr(&k_combine_bwd<W, FP16, kAll, COMPACT>);
}

template <int W, bool FP16>
const void* pick_combine_bwd_stream(int cz)
{
    return cz == kPlan ? fn_ptr(&k_combine_bwd_stream<W, FP16, kPlan>)
           : cz == kPieces ? fn_ptr(&k_combine_bwd_stream<W, FP16, kPieces>)
                           : fn_ptr(&k_combine_bwd_stream<W, FP16, kAll>);
}

cam_status launch_combine_bwd(const CombineBwd& a, void* stream)
{
    const int cz = causal_rule(a);
    const void* fn = nullptr;
    if (CAM_COMBINE_BWD_STREAM && !a.compact && a.g_log2 == 6) {
        // rows of a whole wave or more: one wave per row, no LDS
#define CAM_PICK_BWD_STREAM(Wd)                                                                          \
    if (a.width == Wd)                                                                                   \
        fn = a.fp16 ? pick_combine_bwd_stream<Wd, true>(cz) : pick_combine_bwd_stream<Wd, false>(cz);
        CAM_PICK_BWD_STREAM(16) CAM_PICK_BWD_STREAM(8) CAM_PICK_BWD_STREAM(4) CAM_PICK_BWD_STREAM(2)
#undef CAM_PICK_BWD_STREAM
        const uint32_t wpb = CAM_COMBINE_STREAM_THREADS / 64;
        return launch(fn, a, (a.n_rows + wpb - 1) / wpb, stream, "lse_combine_backward", 0,
                      CAM_COMBINE_STREAM_THREADS);
    }
#define CAM_PICK_BWD(Wd)                                                                                \
    if (a.width == Wd)                                                                                  \
        fn = a.compact ? (a.fp16 ? pick_combine_bwd<Wd, true, true>(cz) : pick_combine_bwd<Wd, false, true>(cz)) \
                       : (a.fp16 ? pick_combine_bwd<Wd, true, false>(cz) : pick_combine_bwd<Wd, false, false>(cz));
    CAM_PICK_BWD(16) CAM_PICK_BWD(8) CAM_PICK_BWD(4) CAM_PICK_BWD(2)
#undef CAM_PICK_BWD
    const uint64_t RB = a.rows_per_tile, G = uint64_t(1) << a.g_log2;
    uint64_t lds = a.compact ? RB * a.P * (8 + 4 + 4 * G) + RB * (8 + 4 + 4)
                             : (2ull * RB * a.P + ((RB + 1) & ~1ull)) * 4 + RB * 8;
    if (a.cu && a.nseq < kCuCache)
        lds += uint64_t(a.nseq + 1) * 4;
    if (lds > 65536)
        return set_error(CAM_ERR_UNSUPPORTED, "lse_combine_backward: a tile's tables need %llu bytes of LDS (at most "
                         "65536)", (unsigned long long)lds);
    return launch(fn, a, a.n_tiles, stream, "lse_combine_backward", lds, a.threads);
}

// The output modes each admission rule is built for: every rule writes at
// the caller's strides; the token-major exchange layout (1) has no causal
// rule; the rank-major varlen shards (2) follow the piece rule.
template <int W, bool FP16, int RF, bool WV>
const void* pick_combine_tiled(int cz, int om)
{
    if (cz == kAll)
        return om == 1 ? fn_ptr(&k_combine<W, FP16, kAll, RF, WV, 1>)
               : om == 0 ? fn_ptr(&k_combine<W, FP16, kAll, RF, WV, 0>) : nullptr;
    if (cz == kPieces)
        return om == 2 ? fn_ptr(&k_combine<W, FP16, kPieces, RF, WV, 2>)
               : om == 0 ? fn_ptr(&k_combine<W, FP16, kPieces, RF, WV, 0>) : nullptr;
    return om == 0 ? fn_ptr(&k_combine<W, FP16, kPlan, RF, WV, 0>) : nullptr;
}

template <int W, bool FP16>
const void* pick_combine_stream(int cz, int om)
{
    if (cz == kAll)
        return om == 1 ? fn_ptr(&k_combine_stream<W, FP16, kAll, 1>)
               : om == 0 ? fn_ptr(&k_combine_stream<W, FP16, kAll, 0>) : nullptr;
    if (cz == kPieces)
        return om == 2 ? fn_ptr(&k_combine_stream<W, FP16, kPieces, 2>)
               : om == 0 ? fn_ptr(&k_combine_stream<W, FP16, kPieces, 0>) : nullptr;
    return om == 0 ? fn_ptr(&k_combine_stream<W, FP16, kPlan, 0>) : nullptr;
}

// Rows of at least 512 bytes (one or more full 64-lane passes) keep two rows
// in flight per lane group; shorter rows, packed several per wave, keep one
// (the lower register count buys occupancy) -- measured on MI355X.  Rows of
// a whole wave or more take the LDS-free row-stream kernel.
template <int W, bool FP16>
const void* pick_combine(int cz, int om, bool wide, bool wave)
{
    if (wave)
        return CAM_COMBINE_STREAM ? pick_combine_stream<W, FP16>(cz, om)
                                  : pick_combine_tiled<W, FP16, kCombineInFlightWave, true>(cz, om);
    return wide ? pick_combine_tiled<W, FP16, 2, false>(cz, om) : pick_combine_tiled<W, FP16, 1, false>(cz, om);
}

cam_status launch_combine(const Combine& a, void* stream)
{
    const bool wide = uint64_t(a.cv) * a.width >= 512;
    const bool wave = a.g_log2 == 6;  // a whole wave per row (implies wide)
    const int cz = causal_rule(a);
    const void* fn = nullptr;
#define CAM_PICK(Wd)                                                                                   \
    if (a.width == Wd)                                                                                 \
        fn = a.fp16 ? pick_combine<Wd, true>(cz, a.out_mode, wide, wave)                               \
                    : pick_combine<Wd, false>(cz, a.out_mode, wide, wave);
    CAM_PICK(16) CAM_PICK(8) CAM_PICK(4) CAM_PICK(2)
#undef CAM_PICK
    if (!fn)
        return CAM_ERR_UNSUPPORTED;
    if (wave && CAM_COMBINE_STREAM) {
        const uint64_t waves = (a.n_rows + CAM_COMBINE_STREAM_ROWS - 1) / CAM_COMBINE_STREAM_ROWS;
        const uint32_t wpb = CAM_COMBINE_STREAM_THREADS / 64;
        return launch(fn, a, (waves + wpb - 1) / wpb, stream, "lse_combine", 0, CAM_COMBINE_STREAM_THREADS);
    }
    // weights [rows][P] (padded to 8 bytes); WAVE: masks [rows], else the
    // compacted offsets [rows][P]; output offsets [rows]; 1/Z or counts [rows]
    const uint64_t RB = a.rows_per_tile;
    uint64_t lds = ((RB * a.P + 1) & ~1ull) * 4 + (wave ? RB : RB * a.P) * 8 + RB * 8 + RB * 4;
    if (a.cu && a.nseq < kCuCache)
        lds += uint64_t(a.nseq + 1) * 4;
    if (lds > 65536)
        return set_error(CAM_ERR_UNSUPPORTED, "lse_combine: a tile's tables need %llu bytes of LDS (at most 65536)",
                         (unsigned long long)lds);
#ifdef CAM_COMBINE_GRID_CAP
    const uint64_t grid = a.n_tiles < CAM_COMBINE_GRID_CAP ? a.n_tiles : CAM_COMBINE_GRID_CAP;
#else
    const uint64_t grid = a.n_tiles;
#endif
    return launch(fn, a, grid, stream, "lse_combine", lds, a.threads);
}

}  // namespace cam
