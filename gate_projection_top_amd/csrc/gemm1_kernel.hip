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
// global memory, four steps' loads issued before their MFMAs.  A operands
// are loaded in the MFMA layout (lane l: row l % 16, k = 8 (l / 16) .. +7 of
// each step); the activations stay in L2.  The weights, read once per call,
// are loaded two steps (128 bytes of each row) at a time so that every load
// covers whole cache lines and can be non-temporal: with lane l = 16 g + n,
// r = n mod 8, h = n / 8, load P brings row r, 16-byte chunk g + 4 h, and
// load Q row 8 + r, chunk g + 4 (1 - h) -- eight full 128-byte lines each.
// The first step's operand (row n, chunk g) is then P for h = 0 and Q for
// h = 1; the second step's (row n, chunk 4 + g) sits in the lane 8 away in
// the same 16-lane row, in P for n < 8 and in Q for n >= 8, so it is the
// other selection rotated by 8 within the row (DPP row_ror:8).  The kernel is
// bound by HBM on the expert weights.
#include "coherent.hpp"
#include "launch.hpp"
#include "route_common.hpp"

namespace gpt {
namespace {

constexpr int kG1Waves = 4;
constexpr int kG1Cols = 16 * kG1Waves;  // output features per workgroup
constexpr int kG1Chunk = 4;             // k-steps whose loads a wave issues together (two line pairs)

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
    // the weight loads P and Q (see the layout above): row and k offset
    const int g = lane >> 4, h = (lane >> 3) & 1;
    const int64_t fp = (int64_t)tile * kG1Cols + wave * 16 + (lane & 7), fq = fp + 8;
    const bool p_ok = fp < a.F, q_ok = fq < a.F;
    const int kp = 8 * (g + 4 * h), kqq = 8 * (g + 4 * (h ^ 1));
    const uint16_t* wpp = a.w1 + (id * a.F + (p_ok ? fp : 0)) * a.D + kp;
    const uint16_t* wpq = a.w1 + (id * a.F + (q_ok ? fq : 0)) * a.D + kqq;

    const bf16x8 zero = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    const int KS = (int)((a.D + 31) >> 5);
    for (int base_ks = 0; base_ks < KS; base_ks += kG1Chunk) {
        bf16x8 av[kG1Chunk], bv[kG1Chunk];
        u32x4 wp[kG1Chunk / 2], wq[kG1Chunk / 2];
#pragma unroll
        for (int c = 0; c < kG1Chunk; ++c) {
            const int k0 = (base_ks + c) * 32;
            const bool in = base_ks + c < KS && (k0 + kq) < a.D;
            av[c] = (in && a_ok) ? load_bf16x8(xp + k0) : zero;
        }
#pragma unroll
        for (int c2 = 0; c2 < kG1Chunk / 2; ++c2) {
            const int k0 = (base_ks + 2 * c2) * 32;  // D % 8 == 0: a lane's 8 values are all in or all out
            wp[c2] = (p_ok && k0 + kp < a.D) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wpp + k0))
                                             : zero4;
            wq[c2] = (q_ok && k0 + kqq < a.D) ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wpq + k0))
                                              : zero4;
        }
#pragma unroll
        for (int c2 = 0; c2 < kG1Chunk / 2; ++c2) {
            const u32x4 first = h ? wq[c2] : wp[c2];
            const u32x4 other = h ? wp[c2] : wq[c2];
            u32x4 second;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                second[e] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)other[e], 0x128, 0xF, 0xF, false);  // row_ror:8
            bv[2 * c2] = __builtin_bit_cast(bf16x8, first);
            bv[2 * c2 + 1] = __builtin_bit_cast(bf16x8, second);
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
