// Double-precision exp for the softmax scores exp(l - max l) of the
// routing (the scoring step of the router: dense_router_decode notes,
// "DenseRouterDecodeKernel"), cheaper than the library's exp: x = k ln2/64 + r
// with |r| <= ln2/128 (Cody-Waite: ln2/64 in a 36-bit and a 53-bit part, so
// that k ln2/64 costs no rounding for |k| < 2^17), exp(r) - 1 from its Taylor
// polynomial of degree 5 (the next term is below 2^-57), 2^(j/64), j = k mod
// 64, as the double pair hi + lo nearest to it, and 2^floor(k/64) by ldexp.
// x is first clamped to [-800, 800] (exp(-800) is 0 in double).  The result
// is within one unit in the last place of exp(x) (checked against exact
// decimal arithmetic by the CPU tests).
//
// On the device the 64 table pairs sit one per lane of the wavefront
// (load_exp2_lane, once per wave) and a lookup is a lane read through the
// LDS crossbar (ds_bpermute); every lane of the wavefront must be active.
// The constants are printed by gen_softmax_exp.py.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt {

constexpr double kExpInvL = 0x1.71547652b82fep+6;  // 64 / ln 2
constexpr double kExpLhi = 0x1.62e42fefa0000p-7;   // ln 2 / 64, leading 36 bits
constexpr double kExpLlo = 0x1.cf79abc9e3b3ap-46;   // ln 2 / 64 - kExpLhi
// 2^(j/64) = hi + lo, j = 0..63
static __device__ const double kExp2Table[64][2] = {
    {0x1.0000000000000p+0, 0x0.0p+0},
    {0x1.02c9a3e778061p+0, -0x1.19083535b085dp-56},
    {0x1.059b0d3158574p+0, 0x1.d73e2a475b465p-55},
    {0x1.0874518759bc8p+0, 0x1.186be4bb284ffp-57},
    {0x1.0b5586cf9890fp+0, 0x1.8a62e4adc610bp-54},
    {0x1.0e3ec32d3d1a2p+0, 0x1.03a1727c57b53p-59},
    {0x1.11301d0125b51p+0, -0x1.6c51039449b3ap-54},
    {0x1.1429aaea92de0p+0, -0x1.32fbf9af1369ep-54},
    {0x1.172b83c7d517bp+0, -0x1.19041b9d78a76p-55},
    {0x1.1a35beb6fcb75p+0, 0x1.e5b4c7b4968e4p-55},
    {0x1.1d4873168b9aap+0, 0x1.e016e00a2643cp-54},
    {0x1.2063b88628cd6p+0, 0x1.dc775814a8495p-55},
    {0x1.2387a6e756238p+0, 0x1.9b07eb6c70573p-54},
    {0x1.26b4565e27cddp+0, 0x1.2bd339940e9d9p-55},
    {0x1.29e9df51fdee1p+0, 0x1.612e8afad1255p-55},
    {0x1.2d285a6e4030bp+0, 0x1.0024754db41d5p-54},
    {0x1.306fe0a31b715p+0, 0x1.6f46ad23182e4p-55},
    {0x1.33c08b26416ffp+0, 0x1.32721843659a6p-54},
    {0x1.371a7373aa9cbp+0, -0x1.63aeabf42eae2p-54},
    {0x1.3a7db34e59ff7p+0, -0x1.5e436d661f5e3p-56},
    {0x1.3dea64c123422p+0, 0x1.ada0911f09ebcp-55},
    {0x1.4160a21f72e2ap+0, -0x1.ef3691c309278p-58},
    {0x1.44e086061892dp+0, 0x1.89b7a04ef80d0p-59},
    {0x1.486a2b5c13cd0p+0, 0x1.3c1a3b69062f0p-56},
    {0x1.4bfdad5362a27p+0, 0x1.d4397afec42e2p-56},
    {0x1.4f9b2769d2ca7p+0, -0x1.4b309d25957e3p-54},
    {0x1.5342b569d4f82p+0, -0x1.07abe1db13cadp-55},
    {0x1.56f4736b527dap+0, 0x1.9bb2c011d93adp-54},
    {0x1.5ab07dd485429p+0, 0x1.6324c054647adp-54},
    {0x1.5e76f15ad2148p+0, 0x1.ba6f93080e65ep-54},
    {0x1.6247eb03a5585p+0, -0x1.383c17e40b497p-54},
    {0x1.6623882552225p+0, -0x1.bb60987591c34p-54},
    {0x1.6a09e667f3bcdp+0, -0x1.bdd3413b26456p-54},
    {0x1.6dfb23c651a2fp+0, -0x1.bbe3a683c88abp-57},
    {0x1.71f75e8ec5f74p+0, -0x1.16e4786887a99p-55},
    {0x1.75feb564267c9p+0, -0x1.0245957316dd3p-54},
    {0x1.7a11473eb0187p+0, -0x1.41577ee04992fp-55},
    {0x1.7e2f336cf4e62p+0, 0x1.05d02ba15797ep-56},
    {0x1.82589994cce13p+0, -0x1.d4c1dd41532d8p-54},
    {0x1.868d99b4492edp+0, -0x1.fc6f89bd4f6bap-54},
    {0x1.8ace5422aa0dbp+0, 0x1.6e9f156864b27p-54},
    {0x1.8f1ae99157736p+0, 0x1.5cc13a2e3976cp-55},
    {0x1.93737b0cdc5e5p+0, -0x1.75fc781b57ebcp-57},
    {0x1.97d829fde4e50p+0, -0x1.d185b7c1b85d1p-54},
    {0x1.9c49182a3f090p+0, 0x1.c7c46b071f2bep-56},
    {0x1.a0c667b5de565p+0, -0x1.359495d1cd533p-54},
    {0x1.a5503b23e255dp+0, -0x1.d2f6edb8d41e1p-54},
    {0x1.a9e6b5579fdbfp+0, 0x1.0fac90ef7fd31p-54},
    {0x1.ae89f995ad3adp+0, 0x1.7a1cd345dcc81p-54},
    {0x1.b33a2b84f15fbp+0, -0x1.2805e3084d708p-57},
    {0x1.b7f76f2fb5e47p+0, -0x1.5584f7e54ac3bp-56},
    {0x1.bcc1e904bc1d2p+0, 0x1.23dd07a2d9e84p-55},
    {0x1.c199bdd85529cp+0, 0x1.11065895048ddp-55},
    {0x1.c67f12e57d14bp+0, 0x1.2884dff483cadp-54},
    {0x1.cb720dcef9069p+0, 0x1.503cbd1e949dbp-56},
    {0x1.d072d4a07897cp+0, -0x1.cbc3743797a9cp-54},
    {0x1.d5818dcfba487p+0, 0x1.2ed02d75b3707p-55},
    {0x1.da9e603db3285p+0, 0x1.c2300696db532p-54},
    {0x1.dfc97337b9b5fp+0, -0x1.1a5cd4f184b5cp-54},
    {0x1.e502ee78b3ff6p+0, 0x1.39e8980a9cc8fp-55},
    {0x1.ea4afa2a490dap+0, -0x1.e9c23179c2893p-54},
    {0x1.efa1bee615a27p+0, 0x1.dc7f486a4b6b0p-54},
    {0x1.f50765b6e4540p+0, 0x1.9d3e12dd8a18bp-54},
    {0x1.fa7c1819e90d8p+0, 0x1.74853f3a5931ep-55},
};

// x = k ln2/64 + r
__host__ __device__ __forceinline__ double exp_reduce(double x, int& k)
{
    x = fmin(fmax(x, -800.0), 800.0);
    const double kd = rint(x * kExpInvL);
    k = (int)kd;
    return fma(-kd, kExpLlo, fma(-kd, kExpLhi, x));
}

// 2^(k/64) exp(r), given the table pair (thi, tlo) of k mod 64
__host__ __device__ __forceinline__ double exp_finish(double r, int k, double thi, double tlo)
{
    double q = fma(r, 1.0 / 120.0, 1.0 / 24.0);
    q = fma(r, q, 1.0 / 6.0);
    q = fma(r, q, 0.5);
    q = fma(r, q, 1.0);
    const double p = r * q;  // exp(r) - 1
    return ldexp(thi + fma(thi, p, tlo), k >> 6);
}

// This lane's table pair: 2^(lane/64) = hi + lo.
struct Exp2Lane {
    double hi, lo;
};

__device__ __forceinline__ Exp2Lane load_exp2_lane()
{
    const int lane = threadIdx.x & 63;
    return Exp2Lane{kExp2Table[lane][0], kExp2Table[lane][1]};
}

__device__ __forceinline__ double lane_read_f64(int byte_addr, double v)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(byte_addr, (int)(uint32_t)u);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(byte_addr, (int)(uint32_t)(u >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// exp(x), every lane of the wavefront active; t: load_exp2_lane()
__device__ __forceinline__ double softmax_exp(double x, const Exp2Lane& t)
{
    int k = 0;
    const double r = exp_reduce(x, k);
    const int a = (k & 63) << 2;
    return exp_finish(r, k, lane_read_f64(a, t.hi), lane_read_f64(a, t.lo));
}

}  // namespace gpt
