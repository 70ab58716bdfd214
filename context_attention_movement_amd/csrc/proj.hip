// proj.hip -- Q/K/V projection whose epilogue writes the head-sharded layout
// of the Ulysses all-to-all directly (FastVideo "[perf] Probe H3 chunked
// all-to-all with direct output slices": fewer passes over local memory by
// writing destination slices in place; here the producer of the scatter
// operand writes them, so the seq->head relayout of Q/K/V disappears).
//
//   out[r][b][t][h'][d] = sum_k x[t][k] * w[(b*H + r*Hp + h')*D + d][k]
//
// x is the P ranks' sequence shards stacked in token order [S][K]; w is the
// fused Q/K/V weight as a linear layer stores it, [N = B*H*D][K]; both are
// K-contiguous, which is the operand layout of the MFMA (a lane holds 8
// consecutive k of one row of A and of one column of B).
//
// Design for gfx950: 256 x 256 output tiles, K in steps of 64 staged through
// LDS (two stages, 16-byte chunks XOR-swizzled by row so the fragment reads
// of 32 consecutive rows spread over the banks), eight waves each owning a
// 128 x 64 sub-tile of v_mfma_f32_32x32x16 blocks (fp32 accumulators), the
// next K step's operands moved global -> LDS directly while the current
// step's MFMAs run.  The epilogue rounds to the payload type and writes each
// output row segment at its head-sharded address.
#include "cam_device.h"

#include <type_traits>

namespace cam {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPM = 256, kPN = 256, kPK = 64;
constexpr int kPStage = (kPM + kPN) * kPK * 2;  // bytes of one LDS stage
// epilogue tile in LDS: rows of 256 payload values padded by 8, so the two
// half-waves of a store (rows 4 apart) fall on different banks
constexpr int kCPitch = kPN + 8;
constexpr int kPLds = (2 * kPStage > kPM * kCPitch * 2) ? 2 * kPStage : kPM * kCPitch * 2;
// waves per workgroup along M and N: 2 x 4, each wave a 128 x 64 sub-tile
// (4 x 2 measures the same within noise; 2 x 2, one wave per SIMD, slower)
// interleave the next k slice's LDS reads with this slice's MFMAs in the
// schedule (1) or leave the order to the compiler (0)
#ifndef CAM_PROJ_INTERLEAVE
#define CAM_PROJ_INTERLEAVE 1
#endif
#ifndef CAM_PROJ_WAVES_M
#define CAM_PROJ_WAVES_M 2
#endif
#ifndef CAM_PROJ_WAVES_N
#define CAM_PROJ_WAVES_N 4
#endif
constexpr int kPWM = CAM_PROJ_WAVES_M, kPWN = CAM_PROJ_WAVES_N;
constexpr int kPThreads = 64 * kPWM * kPWN;
constexpr int kPTM = kPM / kPWM / 32, kPTN = kPN / kPWN / 32;  // 32 x 32 blocks per wave

template <bool FP16>
__device__ __forceinline__ f32x16 mfma_32x32x16(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (FP16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
}

// byte offset of 16-byte chunk c (of 8) of tile row `row` in a [rows][64]
// stage.  LDS serves a 16-byte read of 16 lanes from 64 banks (256 bytes):
// two 128-byte rows share the banks, so the chunk is XOR-ed with (row / 2) % 8
// -- 16 consecutive rows then read 16 distinct bank groups.
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t c)
{
    return row * 128u + ((c ^ ((row >> CAM_PROJ_SWZ_SHIFT) & 7u)) << 4);
}

// The operands move global -> LDS directly (global_load_lds_dwordx4: lane l
// of an instruction writes 16 bytes at the wave's LDS base + 16 l), so no
// registers stage them and no LDS store is issued; the next K step's loads
// fly while the current step's MFMAs run.  Lane l of instruction i of wave w
// fills LDS slot l of the 1 KB block w * per_wave + i: tile row
// 8 * block + l / 8 at chunk position l % 8, i.e. it fetches the logical
// chunk that the swizzle places there.
template <bool FP16>
__global__ __launch_bounds__(kPThreads) void k_proj_direct(Proj a)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
    const uint32_t wm = wave / kPWN, wn = wave % kPWN;
    const uint32_t t = blockIdx.x;
    const uint32_t per_group = a.group_m * a.tiles_n;
    const uint32_t g = t / per_group, first_m = g * a.group_m;
    const uint32_t gsize = min(a.group_m, a.tiles_m - first_m);
    const uint32_t in_g = t - g * per_group;
    const uint32_t tm = first_m + in_g % gsize, tn = in_g / gsize;
    const uint32_t m0 = tm * kPM, n0 = tn * kPN;
    const uint64_t kb = uint64_t(a.K) * 2;

    constexpr int kBlocks = kPM * kPK * 2 / 1024;          // 1 KB blocks per operand per stage
    constexpr int kPerWave = kBlocks / (kPThreads / 64);  // per wave and operand
    const char* ga[kPerWave];
    const char* gb[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
        const uint32_t blk = wave * kPerWave + i;
        const uint32_t row = 8 * blk + (lane >> 3);
        const uint32_t c = (lane & 7u) ^ ((row >> CAM_PROJ_SWZ_SHIFT) & 7u);
        const uint32_t gm = min(m0 + row, a.M - 1);
        ga[i] = static_cast<const char*>(a.x) + gm * kb + c * 16;
        gb[i] = static_cast<const char*>(a.w) + uint64_t(n0 + row) * kb + c * 16;
    }
    auto issue = [&](uint32_t kt, uint32_t stage) {
        char* sa = lds + stage * kPStage;
        char* sb = sa + kPM * kPK * 2;
#pragma unroll
        for (int i = 0; i < kPerWave; ++i) {
            const uint32_t blk = wave * kPerWave + i;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(ga[i] + uint64_t(kt) * kPK * 2),
                                             (__attribute__((address_space(3))) void*)(sa + blk * 1024), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(gb[i] + uint64_t(kt) * kPK * 2),
                                             (__attribute__((address_space(3))) void*)(sb + blk * 1024), 16, 0, 0);
        }
    };

    f32x16 acc[kPTM][kPTN];
#pragma unroll
    for (int i = 0; i < kPTM; ++i)
#pragma unroll
        for (int j = 0; j < kPTN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    const uint32_t nk = a.K / kPK;  // >= 1: the host admits K a positive multiple of 64
    issue(0, 0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const uint32_t fr = lane & 31u, fh = lane >> 5;
    const uint32_t arow = wm * (kPM / kPWM) + fr, brow = wn * (kPN / kPWN) + fr;
    // fragments of one 16-wide k slice; two sets, so the next slice's LDS
    // reads are in flight while the current slice's MFMAs issue
    u32x4 fa[2][kPTM], fb[2][kPTN];
    auto frag = [&](const char* sa, const char* sb, uint32_t ks, int set) {
        const uint32_t c = 2 * ks + fh;
#pragma unroll
        for (int i = 0; i < kPTM; ++i)
            fa[set][i] = *reinterpret_cast<const u32x4*>(sa + swz(arow + i * 32, c));
#pragma unroll
        for (int j = 0; j < kPTN; ++j)
            fb[set][j] = *reinterpret_cast<const u32x4*>(sb + swz(brow + j * 32, c));
    };
    // One K step: the next step's operands are requested first; the barrier
    // that hands the next stage over sits before the last slice's MFMAs, so
    // the next stage's first fragments are read while those MFMAs run.  The
    // last step (LAST) requests and reads nothing more; keeping it a separate
    // copy of the body leaves no join in the loop where the compiler would
    // wait for reads that are not needed yet.
    auto step = [&](uint32_t kt, auto last_tag) {
        constexpr bool LAST = decltype(last_tag)::value;
        const uint32_t cur = kt & 1u;
        if (!LAST)
            issue(kt + 1, cur ^ 1u);
        const char* sa = lds + cur * kPStage;
        const char* sb = sa + kPM * kPK * 2;
#pragma unroll
        for (uint32_t ks = 0; ks < kPK / 16; ++ks) {
            const int set = int(ks & 1u);
            if (ks + 1 < kPK / 16) {
                frag(sa, sb, ks + 1, set ^ 1);
            } else if (!LAST) {
                __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of the next stage have landed
                __syncthreads();                // and everyone's; every read of this stage is done
                const char* na = lds + (cur ^ 1u) * kPStage;
                frag(na, na + kPM * kPK * 2, 0, set ^ 1);
            }
#pragma unroll
            for (int i = 0; i < kPTM; ++i)
#pragma unroll
                for (int j = 0; j < kPTN; ++j)
                    acc[i][j] = mfma_32x32x16<FP16>(fa[set][i], fb[set][j], acc[i][j]);
#if CAM_PROJ_INTERLEAVE
            // spread the next slice's LDS reads between this slice's MFMAs
            if (ks + 1 < kPK / 16) {
#pragma unroll
                for (int u = 0; u < kPTM + kPTN; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x0008, (kPTM * kPTN) / (kPTM + kPTN) > 0 ? (kPTM * kPTN) / (kPTM + kPTN) : 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
                }
            }
#endif
        }
    };
    frag(lds, lds + kPM * kPK * 2, 0, 0);
    for (uint32_t kt = 0; kt + 1 < nk; ++kt)
        step(kt, std::false_type{});
    step(nk - 1, std::true_type{});
    __syncthreads();  // every wave's MFMAs are done with LDS before the epilogue reuses it

    uint16_t* out = static_cast<uint16_t*>(a.out);
    if (a.vec_out) {
        // through LDS: the tile as [256 rows][256 columns] payload values,
        // then 16-byte row segments (8 columns never cross a head block when
        // (H/P)*D is a multiple of 8)
        uint16_t* ct = reinterpret_cast<uint16_t*>(lds);
#pragma unroll
        for (int i = 0; i < kPTM; ++i)
#pragma unroll
            for (int j = 0; j < kPTN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const uint32_t r = wm * (kPM / kPWM) + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                    const uint32_t c = brow + j * 32;
                    const float v = acc[i][j][e];
                    ct[r * kCPitch + c] = FP16 ? __builtin_bit_cast(uint16_t, _Float16(v)) : uint16_t(f32_to_bf16_bits(v));
                }
        __syncthreads();
        constexpr int kVecs = kPM * kPN / 8 / kPThreads;
#pragma unroll
        for (int u = 0; u < kVecs; ++u) {
            const uint32_t q = tid + uint32_t(u) * kPThreads;
            const uint32_t r = q / (kPN / 8), v = q % (kPN / 8);
            const uint32_t m = m0 + r;
            if (m < a.M) {
                const uint32_t n = n0 + v * 8;
                const uint32_t b = fdiv(n, a.div_HD);
                const uint32_t rem = n - b * a.HD;
                const uint32_t rr = fdiv(rem, a.div_HpD);
                const uint32_t cc = rem - rr * a.HpD;
                const uint64_t off = ((uint64_t(rr) * a.B + b) * a.S + m) * a.HpD + cc;
                *reinterpret_cast<u32x4*>(out + off) = *reinterpret_cast<const u32x4*>(ct + r * kCPitch + v * 8);
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < kPTN; ++j) {
        const uint32_t n = n0 + brow + j * 32;
        const uint32_t b = fdiv(n, a.div_HD);
        const uint32_t rem = n - b * a.HD;
        const uint32_t r = fdiv(rem, a.div_HpD);
        const uint32_t cc = rem - r * a.HpD;
        const uint64_t base = (uint64_t(r) * a.B + b) * a.S;
#pragma unroll
        for (int i = 0; i < kPTM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t m = m0 + wm * (kPM / kPWM) + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                if (m < a.M) {
                    const float v = acc[i][j][e];
                    const uint16_t h = FP16 ? __builtin_bit_cast(uint16_t, _Float16(v)) : uint16_t(f32_to_bf16_bits(v));
                    out[(base + m) * a.HpD + cc] = h;
                }
            }
    }
}

cam_status launch_proj(const Proj& a, void* stream)
{
    const void* fn = a.fp16 ? reinterpret_cast<const void*>(&k_proj_direct<true>)
                            : reinterpret_cast<const void*>(&k_proj_direct<false>);
    // two 64 KB stages (and the padded epilogue tile): above the default
    // dynamic-LDS limit of a launch
    static thread_local const void* opted[2] = {nullptr, nullptr};
    if (opted[a.fp16] != fn) {
        const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kPLds);
        if (e != hipSuccess)
            return set_error(CAM_ERR_HIP, "qkv_projection_head_sharded: %s", hipGetErrorString(e));
        opted[a.fp16] = fn;
    }
    return launch(fn, a, uint64_t(a.tiles_m) * a.tiles_n, stream, "qkv_projection_head_sharded", kPLds, kPThreads);
}

}  // namespace cam
