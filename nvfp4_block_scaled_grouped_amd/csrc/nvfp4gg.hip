// nvfp4gg.hip -- NVFP4 block-scaled grouped GEMM for MI355X (gfx950).
//
// C_i = A_i . B_i^T per group, A/B packed FP4 E2M1 with one E4M3 scale per 16
// K of a row, fp32 accumulation, fp16 output (kernelindex page
// kernelbot-nvfp4-group-gemm-444497, kernel-source header comment; page
// kernelbot-nvfp4-group-gemm-505431, custom_kernel_fallback).  The C ABI is
// declared in include/nvfp4gg.h.
//
// Design (gfx950 first; the pages' Blackwell kernels are prior art only):
//   * Scale resolution: every A and B element is dequantised in registers to
//     fp16 as e2m1(code) * e4m3(scale).  That product has at most 6
//     significant bits and lies in [2^-10, 2688], so fp16 holds it exactly,
//     and the fp16 x fp16 products inside the MFMA are exact in fp32.  The
//     contraction then runs on v_mfma_f32_16x16x32_f16 with fp32 accumulation.
//     (CDNA4's block-scaled f8f6f4 MFMA takes power-of-two E8M0 scales per 32
//     K; it cannot carry an E4M3 mantissa per 16 K, and no 8-bit operand
//     format holds a 6-bit significand.)
//   * Dequant: v_cvt_scalef32_pk_f16_fp4 turns two FP4 codes into two fp16
//     (scale operand 1.0), then v_pk_mul_f16 multiplies by the E4M3 scale
//     converted to fp16 (exact: E4M3 is a subset of fp16).
//   * K order: the sum over K is order-free, so each 16-lane group q of a
//     wave owns a contiguous quarter of every 256-wide K step (32 bytes per
//     row = two 16-byte loads, one 4-byte scale load).  In MFMA k-step j the
//     lane feeds the 8 codes of dword j of its quarter; A and B use the same
//     assignment, so the pairs (a_k, b_k) meet in the same MFMA slot.
//   * Accumulation is hierarchical: each 512-K stretch accumulates into a
//     fresh fp32 tile that is then added into the running tile, which keeps
//     the rounding error of long K sums small next to outputs near zero.
//   * Loads are raw buffer loads with the exact byte size as the range, so
//     rows past M_i or N_i read as zero without branches.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>

#include "nvfp4gg.h"

namespace {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef int i4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWave * kWavesPerBlock;
constexpr int kBM = 64;                       // rows of A per block (4 x 16)
constexpr int kWN = 64;                       // columns of B per wave (4 x 16)
constexpr int kBN = kWN * kWavesPerBlock;     // columns of B per block
constexpr int kKStep = 256;                   // K per pipeline step
constexpr int kFlushSteps = 2;                // K steps per partial accumulation
constexpr int kMaxGroupsPerLaunch = 32;
constexpr uint32_t kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

struct GroupDesc {
    const uint8_t* A;
    const uint8_t* B;
    const uint8_t* SFA;
    const uint8_t* SFB;
    uint16_t* C;
    int M, N, K;
    int item_begin;   // first work item of this group within the launch
    int mblocks;      // ceil(M / kBM)
    int nblocks;      // ceil(N / kBN)
    int pad0, pad1;
};

struct LaunchArgs {
    GroupDesc g[kMaxGroupsPerLaunch];
    int ngroups;
    int total_items;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             (int)kBufferFlags);
}

// Eight FP4 codes (one dword, nibble order) times a shared fp16 scale.
__device__ __forceinline__ h8_t dequant8(uint32_t packed, _Float16 s)
{
    const h2_t s2 = {s, s};
    const h2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 0) * s2;
    const h2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 1) * s2;
    const h2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 2) * s2;
    const h2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(packed, 1.0f, 3) * s2;
    return h8_t{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// One 16-row operand fragment for one 256-wide K step, as one lane holds it:
// 32 bytes of codes (8 dwords, 64 consecutive K) and their 4 scale bytes.
struct Frag {
    i4_t lo, hi;
    uint32_t sc;
};

__device__ __forceinline__ Frag load_frag(__amdgpu_buffer_rsrc_t codes, __amdgpu_buffer_rsrc_t scales,
                                          uint32_t code_off, uint32_t scale_off)
{
    Frag f;
    f.lo = __builtin_bit_cast(i4_t, __builtin_amdgcn_raw_buffer_load_b128(codes, code_off, 0, 0));
    f.hi = __builtin_bit_cast(i4_t, __builtin_amdgcn_raw_buffer_load_b128(codes, code_off + 16, 0, 0));
    f.sc = __builtin_amdgcn_raw_buffer_load_b32(scales, scale_off, 0, 0);
    return f;
}

__device__ __forceinline__ uint32_t frag_dword(const Frag& f, int j)
{
    return (uint32_t)(j < 4 ? f.lo[j & 3] : f.hi[j & 3]);
}

// Scales of k-steps (0,1), (2,3), (4,5), (6,7) are bytes 0..3 of f.sc.
__device__ __forceinline__ void frag_scales(const Frag& f, _Float16 out[4])
{
    const h2_t s01 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sc, 1.0f, false);
    const h2_t s23 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sc, 1.0f, true);
    out[0] = s01.x;
    out[1] = s01.y;
    out[2] = s23.x;
    out[3] = s23.y;
}

__global__ __launch_bounds__(kThreads) void nvfp4_group_gemm_kernel(const LaunchArgs args)
{
    const int item = blockIdx.x;
    int gi = 0;
    for (int i = 1; i < args.ngroups; ++i)
        if (item >= args.g[i].item_begin) gi = i;
    const GroupDesc& G = args.g[gi];

    const int li = item - G.item_begin;
    const int mb = li % G.mblocks;
    const int nb = li / G.mblocks;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x % kWave;
    const int r16 = lane & 15;   // row within a 16-row fragment
    const int q = lane >> 4;     // K quarter owned by this lane group

    const int M = G.M, N = G.N, K = G.K;
    const int m0 = mb * kBM;
    const int n0 = nb * kBN + wave * kWN;
    const uint32_t row_bytes = (uint32_t)K / 2;
    const uint32_t row_scales = (uint32_t)K / 16;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(G.A, (uint32_t)M * row_bytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(G.B, (uint32_t)N * row_bytes);
    const __amdgpu_buffer_rsrc_t rSA = make_rsrc(G.SFA, (uint32_t)M * row_scales);
    const __amdgpu_buffer_rsrc_t rSB = make_rsrc(G.SFB, (uint32_t)N * row_scales);

    uint32_t offA[4], offSA[4], offB[4], offSB[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const uint32_t ra = (uint32_t)(m0 + 16 * f + r16);
        const uint32_t rb = (uint32_t)(n0 + 16 * f + r16);
        offA[f] = ra * row_bytes + 32u * q;
        offSA[f] = ra * row_scales + 4u * q;
        offB[f] = rb * row_bytes + 32u * q;
        offSB[f] = rb * row_scales + 4u * q;
    }

    // acc[i][j]: output tile with B fragment i (16 columns of C) as the MFMA
    // A operand and A fragment j (16 rows of C) as the MFMA B operand.
    f4_t acc[4][4];
    f4_t part[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            acc[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};
            part[i][j] = f4_t{0.f, 0.f, 0.f, 0.f};
        }

    Frag fa[4], fb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        fa[f] = load_frag(rA, rSA, offA[f], offSA[f]);
        fb[f] = load_frag(rB, rSB, offB[f], offSB[f]);
    }

    int step = 0;
    for (int kb = 0; kb < K; kb += kKStep, ++step) {
        // Prefetch the next step (range-checked loads; unused past K).
        Frag na[4], nbf[4];
        const uint32_t nk_bytes = (uint32_t)(kb + kKStep) / 2;
        const uint32_t nk_scales = (uint32_t)(kb + kKStep) / 16;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            na[f] = load_frag(rA, rSA, offA[f] + nk_bytes, offSA[f] + nk_scales);
            nbf[f] = load_frag(rB, rSB, offB[f] + nk_bytes, offSB[f] + nk_scales);
        }

        _Float16 sa[4][4], sb[4][4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            frag_scales(fa[f], sa[f]);
            frag_scales(fb[f], sb[f]);
        }

#pragma unroll
        for (int j = 0; j < 8; ++j) {
            h8_t av[4], bv[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                av[f] = dequant8(frag_dword(fa[f], j), sa[f][j >> 1]);
                bv[f] = dequant8(frag_dword(fb[f], j), sb[f][j >> 1]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    part[i][jj] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv[i], av[jj], part[i][jj], 0, 0, 0);
        }

        if ((step % kFlushSteps) == kFlushSteps - 1 || kb + kKStep >= K) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    acc[i][jj] += part[i][jj];
                    part[i][jj] = f4_t{0.f, 0.f, 0.f, 0.f};
                }
        }

#pragma unroll
        for (int f = 0; f < 4; ++f) {
            fa[f] = na[f];
            fb[f] = nbf[f];
        }
    }

    // Epilogue: lane holds C[m][n .. n+3] for m = m0 + 16 jj + r16,
    // n = n0 + 16 i + 4 q; fp32 -> fp16 round-to-nearest-even (overflow to inf).
    uint16_t* C = G.C;
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        const int m = m0 + 16 * jj + r16;
        if (m >= M) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = n0 + 16 * i + 4 * q;
            if (n >= N) continue;
            const f4_t v = acc[i][jj];
            const _Float16 h[4] = {(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
            uint16_t* dst = C + (size_t)m * N + n;
            if (vec_ok && n + 3 < N) {
                uint2 w;
                w.x = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
                w.y = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
                *reinterpret_cast<uint2*>(dst) = w;
            } else {
                for (int e = 0; e < 4 && n + e < N; ++e)
                    dst[e] = __builtin_bit_cast(uint16_t, h[e]);
            }
        }
    }
}

// Dequantisation alone, through the same fragment path as the GEMM: one
// thread per 64 consecutive codes of a row (one quarter-step of a lane),
// i.e. 8 dwords of codes and the 4 scale bytes that cover them.  Blocks past
// the end of the row are skipped.
__global__ __launch_bounds__(256) void nvfp4_dequant_kernel(int rows, int K, const uint8_t* X,
                                                            const uint8_t* SFX, h8_t* out)
{
    const int blocks = K / 16;                 // scale blocks per row
    const int quads = (blocks + 3) / 4;        // 4-block pieces per row
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t >= (int64_t)rows * quads) return;
    const int64_t r = t / quads;
    const int b0 = (int)(t % quads) * 4;
    const int nb = blocks - b0 < 4 ? blocks - b0 : 4;

    Frag f;
    uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    uint32_t sc = 0;
    const uint32_t* xrow = reinterpret_cast<const uint32_t*>(X + r * (K / 2));
    for (int b = 0; b < nb; ++b) {
        w[2 * b] = xrow[2 * (b0 + b)];
        w[2 * b + 1] = xrow[2 * (b0 + b) + 1];
        sc |= (uint32_t)SFX[r * blocks + b0 + b] << (8 * b);
    }
    f.lo = i4_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    f.hi = i4_t{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    f.sc = sc;
    _Float16 s[4];
    frag_scales(f, s);
    h8_t* orow = out + r * (K / 8);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (j < 2 * nb) orow[2 * b0 + j] = dequant8(frag_dword(f, j), s[j >> 1]);
}

thread_local std::string g_last_error;

int fail(int code, const std::string& msg)
{
    g_last_error = msg;
    return code;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace

extern "C" const char* nvfp4_group_gemm_last_error(void) { return g_last_error.c_str(); }

extern "C" int nvfp4_group_gemm_version(void) { return 1; }

extern "C" int nvfp4_group_gemm(int g, const int* M, const int* N, const int* K,
                                const void* const* A_ptrs, const void* const* B_ptrs,
                                const void* const* SFA_ptrs, const void* const* SFB_ptrs,
                                void* const* C_ptrs, void* stream)
{
    g_last_error.clear();
    if (g <= 0) return fail(NVFP4GG_INVALID_ARG, "g must be >= 1");
    if (!M || !N || !K || !A_ptrs || !B_ptrs || !SFA_ptrs || !SFB_ptrs || !C_ptrs)
        return fail(NVFP4GG_INVALID_ARG, "a size or pointer array is NULL");
    for (int i = 0; i < g; ++i) {
        const std::string gs = "group " + std::to_string(i) + ": ";
        if (M[i] < 0 || N[i] < 0 || K[i] < 0) return fail(NVFP4GG_INVALID_ARG, gs + "negative size");
        if (K[i] % 16 != 0) return fail(NVFP4GG_INVALID_ARG, gs + "K must be a multiple of 16");
        if (M[i] == 0 || N[i] == 0) continue;
        if (!C_ptrs[i] || !aligned16(C_ptrs[i]))
            return fail(NVFP4GG_INVALID_ARG, gs + "C pointer is NULL or not 16-byte aligned");
        if (K[i] == 0) continue;
        const void* ops[4] = {A_ptrs[i], B_ptrs[i], SFA_ptrs[i], SFB_ptrs[i]};
        for (const void* p : ops)
            if (!p || !aligned16(p))
                return fail(NVFP4GG_INVALID_ARG, gs + "an operand pointer is NULL or not 16-byte aligned");
        if (K[i] % kKStep != 0)
            return fail(NVFP4GG_UNSUPPORTED, gs + "this kernel needs K % 256 == 0");
        // Byte offsets of the buffer loads are 32-bit and may run one block
        // past the last row.
        const int64_t rows = (int64_t)(M[i] > N[i] ? M[i] : N[i]) + kBN;
        if (rows * (K[i] / 2) >= ((int64_t)1 << 31))
            return fail(NVFP4GG_UNSUPPORTED, gs + "operand larger than 2 GiB");
    }

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    LaunchArgs args;
    int gi = 0;
    while (gi < g) {
        std::memset(&args, 0, sizeof(args));
        int items = 0;
        int n = 0;
        for (; gi < g && n < kMaxGroupsPerLaunch; ++gi) {
            if (M[gi] == 0 || N[gi] == 0) continue;
            GroupDesc& d = args.g[n++];
            d.A = static_cast<const uint8_t*>(A_ptrs[gi]);
            d.B = static_cast<const uint8_t*>(B_ptrs[gi]);
            d.SFA = static_cast<const uint8_t*>(SFA_ptrs[gi]);
            d.SFB = static_cast<const uint8_t*>(SFB_ptrs[gi]);
            d.C = static_cast<uint16_t*>(C_ptrs[gi]);
            d.M = M[gi];
            d.N = N[gi];
            d.K = K[gi];
            d.item_begin = items;
            d.mblocks = ceil_div(M[gi], kBM);
            d.nblocks = ceil_div(N[gi], kBN);
            items += d.mblocks * d.nblocks;
        }
        if (n == 0) continue;
        args.ngroups = n;
        args.total_items = items;
        hipLaunchKernelGGL(nvfp4_group_gemm_kernel, dim3(items), dim3(kThreads), 0, s, args);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return fail(NVFP4GG_HIP_ERROR, std::string("kernel launch failed: ") + hipGetErrorString(e));
    }
    return NVFP4GG_OK;
}

extern "C" int nvfp4_dequant_f16(int rows, int K, const void* X, const void* SFX, void* out, void* stream)
{
    g_last_error.clear();
    if (rows < 0 || K < 0) return fail(NVFP4GG_INVALID_ARG, "negative size");
    if (K % 16 != 0) return fail(NVFP4GG_INVALID_ARG, "K must be a multiple of 16");
    if (rows == 0 || K == 0) return NVFP4GG_OK;
    if (!X || !SFX || !out || !aligned16(X) || !aligned16(SFX) || !aligned16(out))
        return fail(NVFP4GG_INVALID_ARG, "a pointer is NULL or not 16-byte aligned");
    const int64_t total = (int64_t)rows * ((K / 16 + 3) / 4);
    if (total > ((int64_t)1 << 31) - 256) return fail(NVFP4GG_UNSUPPORTED, "too many elements");
    const int nblk = (int)((total + 255) / 256);
    hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3(nblk), dim3(256), 0,
                       reinterpret_cast<hipStream_t>(stream), rows, K,
                       static_cast<const uint8_t*>(X), static_cast<const uint8_t*>(SFX),
                       static_cast<h8_t*>(out));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail(NVFP4GG_HIP_ERROR, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return NVFP4GG_OK;
}
