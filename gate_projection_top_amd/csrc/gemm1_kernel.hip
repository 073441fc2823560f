// Expert GEMM1 on the unique-route table (b70 lab MTP1 M=2 note, "Why
// literal source-direct GEMM1 is not funded": with identical (token, expert)
// routes deduplicated upstream, each expert has the affine rows [token0],
// [token1] or [token0, token1], and the table produced by the router is
// consumed by the GEMMs).  Unique expert u (id unique_ids[u]) multiplies the
// rows of the tokens in token_mask[u] by its weights w1[id] ([F, D]) once,
// however many tokens picked it:
//   out[row(u, t), f] = bf16( fp32 sum over d of x[t, d] * w1[id, f, d] ),
// row(u, t) = (tokens of the unique experts before u) + (tokens of u below
// t): the compact layout the gather reads.
//
// Layout: a workgroup is one unique expert's 64 output features; each of its
// four waves owns 16 of them and runs over all of D in 32-wide MFMA steps
// (v_mfma_f32_16x16x32_bf16): B = 16 weight rows, A = the expert's tokens (at
// most 16, one per A row; the rest zero).  Operands come straight from
// global memory in the MFMA layout (lane l: row / column l % 16, k =
// 8 (l / 16) .. +7 of each step), eight steps' loads issued before their
// MFMAs.  Every weight byte is read once per call; the activations stay in
// L2.  The kernel is bound by HBM on the expert weights.
#include "coherent.hpp"
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {
namespace {

constexpr int kG1Waves = 4;
constexpr int kG1Cols = 16 * kG1Waves;  // output features per workgroup
constexpr int kG1Chunk = 8;             // k-steps whose loads a wave issues together

__global__ __launch_bounds__(kG1Waves * kWave) void expert_gemm1_kernel(Gemm1Launch a)
{
    const int tiles = (int)((a.F + kG1Cols - 1) / kG1Cols);
    const int u = blockIdx.x / tiles;  // unique-expert slot
    const int tile = blockIdx.x % tiles;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;

    const int slots = a.M * a.k;  // <= 64
    int n = *a.unique_count;
    n = n < 0 ? 0 : (n > slots ? slots : n);
    if (u >= n) return;  // workgroup-uniform
    const int64_t id = a.unique_ids[u];
    if (id < 0 || id >= a.E) return;
    const uint32_t tokens_all = (a.M >= 32) ? 0xffffffffu : ((1u << a.M) - 1u);
    // this expert's tokens and its first compact row (tokens of earlier experts)
    const uint32_t mask = (uint32_t)a.token_mask[u] & tokens_all;
    const uint32_t before = lane < u ? (uint32_t)__builtin_popcount((uint32_t)a.token_mask[lane] & tokens_all) : 0u;
    int base = (int)before;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) base += __shfl_xor(base, off);
    const int ntok = __builtin_popcount(mask);

    // A row r (= lane % 16): the r-th token of the mask, if any
    const int r = lane & 15;
    int tok = -1;
    {
        uint32_t m = mask;
        for (int q = 0; q < r && m; ++q) m &= m - 1u;  // drop the r lowest tokens
        tok = m ? __builtin_ctz(m) : -1;
    }
    const int kq = (lane >> 4) * 8;  // this lane's 8 of each step's 32 k
    const int64_t f = (int64_t)tile * kG1Cols + wave * 16 + (lane & 15);  // B column = output feature
    const bool a_ok = tok >= 0;
    const bool b_ok = f < a.F;
    const uint16_t* xp = a.x + (int64_t)(a_ok ? tok : 0) * a.D + kq;
    const uint16_t* wp = a.w1 + (id * a.F + (b_ok ? f : 0)) * a.D + kq;

    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int KS = (int)((a.D + 31) >> 5);
    for (int base_ks = 0; base_ks < KS; base_ks += kG1Chunk) {
        bf16x8 av[kG1Chunk], bv[kG1Chunk];
#pragma unroll
        for (int c = 0; c < kG1Chunk; ++c) {
            const int k0 = (base_ks + c) * 32;
            const bool in = base_ks + c < KS && (k0 + kq) < a.D;
            av[c] = (in && a_ok) ? load_bf16x8(xp + k0) : zero;
            bv[c] = (in && b_ok) ? load_bf16x8(wp + k0) : zero;
        }
#pragma unroll
        for (int c = 0; c < kG1Chunk; ++c)
            if (base_ks + c < KS) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[c], bv[c], acc, 0, 0, 0);
    }
    // C layout: lane holds A rows (token ranks) 4 (lane / 16) + i, column lane % 16
    if (b_ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rank = 4 * (lane >> 4) + i;
            if (rank < ntok)
                a.out[(int64_t)(base + rank) * a.F + f] = __builtin_bit_cast(uint16_t, (__bf16)acc[i]);
        }
    }
}

}  // namespace

hipError_t launch_gemm1(const Gemm1Launch& a, hipStream_t stream)
{
    const int64_t tiles = (a.F + kG1Cols - 1) / kG1Cols;
    const int64_t blocks = (int64_t)a.M * a.k * tiles;
    hipLaunchKernelGGL(expert_gemm1_kernel, dim3((unsigned)blocks), dim3(kG1Waves * kWave), 0, stream, a);
    return hipGetLastError();
}

}  // namespace gpt
