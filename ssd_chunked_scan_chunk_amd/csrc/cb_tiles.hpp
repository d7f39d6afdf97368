// cb_tiles.hpp -- the C B^T tiles of the backward's da kernel, as a device
// routine that any kernel of the library can run on a workgroup it spares.
#pragma once

#include "mfma_util.hpp"
#include "ssd_launch.hpp"

namespace ssd {

// C B^T tiles of every chunk, once per group (the head-independent factor of
// the backward's da kernel, whose masked term is built from the products
// (dY_i . X_j)(C_i . B_j)): tile (I, J), J <= I, of chunk c is C_I B_J^T
// over the chunk's 32-row tiles (rows past a ragged end zero), formed on MFMA
// from the bf16 inputs and stored in the accumulator layout, 16 floats per
// lane: cbt[b][c][g][I(I+1)/2 + J][lane][16].  One wavefront per tile.
template <int N>
__device__ __forceinline__ void cb_tile(const CbJob& j, int b, int64_t c, int g, int t, int lane)
{
    const u16* Bm = static_cast<const u16*>(j.B);
    const u16* Cm = static_cast<const u16*>(j.C);
    const int nI = j.Q / 32, nt = nI * (nI + 1) / 2;
    const int l32 = lane & 31, g2 = lane >> 5;
    const int64_t t0 = c * j.Q;
    const int Lc = (int)((j.L - t0 < j.Q) ? (j.L - t0) : j.Q);
    int I = 0;
    while ((I + 1) * (I + 2) / 2 <= t) ++I;
    const int J = t - I * (I + 1) / 2;
    const int irow = 32 * I + l32, jrow = 32 * J + l32;
    bf16x8 cf[N / 16], bb[N / 16];
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u}, w = {0u, 0u, 0u, 0u};
        if (irow < Lc) v = *reinterpret_cast<const u32x4*>(Cm + (((int64_t)b * j.L + t0 + irow) * j.G + g) * N + 16 * ks + 8 * g2);
        if (jrow < Lc) w = *reinterpret_cast<const u32x4*>(Bm + (((int64_t)b * j.L + t0 + jrow) * j.G + g) * N + 16 * ks + 8 * g2);
        cf[ks] = as_bf16x8(v);
        bb[ks] = as_bf16x8(w);
    }
    f32x16 CB = zero16();
#pragma unroll
    for (int ks = 0; ks < N / 16; ++ks) CB = mfma32(cf[ks], bb[ks], CB);
    float4* o = reinterpret_cast<float4*>(j.cbt + ((((int64_t)b * j.nc + c) * j.G + g) * nt + t) * 1024 + lane * 16);
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = make_float4(CB[4 * k], CB[4 * k + 1], CB[4 * k + 2], CB[4 * k + 3]);
}

// workgroup wi of the cb tiles with W wavefronts per workgroup: ceil(tiles / W)
// workgroups per (batch, chunk, group) item, wave w taking one tile
template <int N, int W>
__device__ __forceinline__ void cb_tiles_wg(const CbJob& j, int64_t wi, int wave, int lane)
{
    const int nI = j.Q / 32, nt = nI * (nI + 1) / 2;
    const int tbs = (nt + W - 1) / W;
    const int64_t item = wi / tbs;
    const int t = (int)(wi - item * tbs) * W + wave;
    if (t >= nt || item >= (int64_t)j.Bz * j.nc * j.G) return;
    const int g = (int)(item % j.G);
    const int64_t c = (item / j.G) % j.nc;
    const int b = (int)(item / j.G / j.nc);
    cb_tile<N>(j, b, c, g, t, lane);
}

// workgroups the tiles take with `waves` wavefronts per workgroup
__host__ __device__ inline int64_t cb_workgroups(const CbJob& j, int waves) {
    const int64_t nI = j.Q / 32, nt = nI * (nI + 1) / 2;
    return (int64_t)j.Bz * j.nc * j.G * ((nt + waves - 1) / waves);
}

}  // namespace ssd
