// Several positives per entry for the sigmoid form.
//
// An entry of the batch may carry several positives besides its own pair
// (UForm README, "Multimodal Perception from 64 to 1024 Dimensions", the
// training-stack paragraph on loader-side properties); each listed cell takes
// the label z = +1.  The dense backward passes leave every listed cell out of
// their band operands and sums (as they do the row's own positive), so this
// pass gives each listed cell, in FP32, its whole positive-label loss
// softplus(-l^p) with l = t cos + b, and its whole residual
// g^p = (sigma(l^p) - 1) / den = -sigma(-l^p) / den.  Summing sigma(l) in a 16-bit
// band operand and subtracting 1 afterwards would lose a confident positive's
// small residual to the operand's rounding.  The row gradient takes g^p
// through the prefix normalisation:
//
//   dx_o[:w_p] += c_p sigma(-l^p) (y_i[:w_p] |x_o^p|^-1 |y_i^p|^-1 - cos^p x_o[:w_p] |x_o^p|^-2)
//
// with c_p = -mirror (w_p / W) t / den.  One wave owns one outer row and walks
// its list in order, so every sum has a fixed order and no atomics are needed.
// The lists are sparse (a few cells per row against the N of the dense pass):
// the pass is a gather of listed rows, bound by HBM and latency, not by MFMA.

#include <hip/hip_runtime.h>

#include "common.h"

namespace uform {
namespace {

// Sum over the wave, in every lane, without LDS round trips: quad permutes (lanes 1 and 2 apart),
// the half-row and row mirrors (the other quad, the other half-row), then the 16-lane and 32-lane
// swaps add the partner row and the partner half-wave.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wsum(float v) {
    v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_mov<0x141>(v);  // row_half_mirror
    v += dpp_mov<0x140>(v);  // row_mirror
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(h[0]) + __uint_as_float(h[1]);
}

// 16 BF16 values (32 bytes, 16-byte aligned) widened to FP32.
__device__ __forceinline__ void load16(const u16 *p, float v[16]) {
    const uint4 a = *(const uint4 *)p, b = *(const uint4 *)(p + 8);
    const unsigned int w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        v[2 * c] = __uint_as_float(w[c] << 16);
        v[2 * c + 1] = __uint_as_float(w[c] & 0xffff0000u);
    }
}

// Lane l holds elements 16 l .. 16 l + 15 of each 1024-wide segment of a row (NSEG segments:
// D <= 1024 NSEG); waves walk the outer rows blockIdx.x * 4 + wave, stepping by the grid.
template <int NSEG>
__global__ __launch_bounds__(256) void k_pos(PosArgs a) {
    __shared__ float red[4][3 * kMaxP];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int P = a.pf.n, D = a.D;
    int d0[NSEG], pl[NSEG];  // segment g: first element, narrowest prefix covering it (P: none)
    bool act[NSEG];
#pragma unroll
    for (int g = 0; g < NSEG; ++g) {
        d0[g] = 16 * lane + 1024 * g;
        act[g] = d0[g] < D;
        pl[g] = P;
        for (int p = P - 1; p >= 0; --p)
            if (d0[g] < a.pf.w[p]) pl[g] = p;
    }
    // sums over this wave's cells (wave-uniform): softplus(-l^p), sigma(-l^p) cos^p, sigma(-l^p)
    float ls[kMaxP], cs[kMaxP], gs[kMaxP];
#pragma unroll
    for (int p = 0; p < kMaxP; ++p) ls[p] = cs[p] = gs[p] = 0.f;

    for (int64_t o = (int64_t)blockIdx.x * 4 + wave; o < a.NO; o += (int64_t)gridDim.x * 4) {
        const int e0 = a.ptr[o], e1 = a.ptr[o + 1];
        if (e0 >= e1) continue;
        float xv[NSEG][16];
#pragma unroll
        for (int g = 0; g < NSEG; ++g) {
            if (act[g])
                load16(a.x + o * D + d0[g], xv[g]);
            else
                for (int c = 0; c < 16; ++c) xv[g][c] = 0.f;
        }
        float ix[kMaxP];
        for (int p = 0; p < P; ++p) ix[p] = a.invx[p * a.NO + o];
        float acc[NSEG][16];
#pragma unroll
        for (int g = 0; g < NSEG; ++g)
#pragma unroll
            for (int c = 0; c < 16; ++c) acc[g][c] = 0.f;
        float xc[NSEG];  // per segment: sum over cells and covering prefixes of c_p sigma(-l^p) cos^p |x^p|^-2
#pragma unroll
        for (int g = 0; g < NSEG; ++g) xc[g] = 0.f;
        for (int e = e0; e < e1; ++e) {
            const int64_t i = a.idx[e];
            float yv[NSEG][16], part[NSEG];
#pragma unroll
            for (int g = 0; g < NSEG; ++g) {
                if (act[g])
                    load16(a.y + i * D + d0[g], yv[g]);
                else
                    for (int c = 0; c < 16; ++c) yv[g][c] = 0.f;
                part[g] = 0.f;
#pragma unroll
                for (int c = 0; c < 16; ++c) part[g] = fmaf(xv[g][c], yv[g][c], part[g]);
            }
            float yc[NSEG];  // per segment: sum over covering prefixes of c_p sigma(-l^p) |x^p|^-1 |y^p|^-1
#pragma unroll
            for (int g = 0; g < NSEG; ++g) yc[g] = 0.f;
            for (int p = 0; p < P; ++p) {
                float mine = 0.f;
#pragma unroll
                for (int g = 0; g < NSEG; ++g) mine += d0[g] < a.pf.w[p] ? part[g] : 0.f;
                const float dot = wsum(mine);
                const float iy = a.invy[p * a.NI + i];
                const float cosv = dot * ix[p] * iy;
                const float l = fmaf(a.t, cosv, a.b);
                // sigma(-l) = 1 / (1 + e^l) (e^l = inf gives 0); softplus(-l) = max(-l, 0) + log1p(e^-|l|)
                const float sn = 1.0f / (1.0f + expf(l));
                ls[p] += fmaxf(-l, 0.f) + log1pf(expf(-fabsf(l)));
                cs[p] = fmaf(sn, cosv, cs[p]);
                gs[p] += sn;
                const float c = a.gc[p] * sn;
#pragma unroll
                for (int g = 0; g < NSEG; ++g)
                    if (p >= pl[g]) {
                        yc[g] = fmaf(c, ix[p] * iy, yc[g]);
                        xc[g] = fmaf(c, cosv * ix[p] * ix[p], xc[g]);
                    }
            }
#pragma unroll
            for (int g = 0; g < NSEG; ++g)
#pragma unroll
                for (int c = 0; c < 16; ++c) acc[g][c] = fmaf(yc[g], yv[g][c], acc[g][c]);
        }
#pragma unroll
        for (int g = 0; g < NSEG; ++g) {
            if (a.out && act[g] && pl[g] < P) {
                float4 *dst = (float4 *)(a.out + o * D + d0[g]);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    float4 v = dst[c];
                    v.x += acc[g][4 * c] - xc[g] * xv[g][4 * c];
                    v.y += acc[g][4 * c + 1] - xc[g] * xv[g][4 * c + 1];
                    v.z += acc[g][4 * c + 2] - xc[g] * xv[g][4 * c + 2];
                    v.w += acc[g][4 * c + 3] - xc[g] * xv[g][4 * c + 3];
                    dst[c] = v;
                }
            }
        }
    }
    if (!a.parts) return;
    if (lane == 0)
        for (int p = 0; p < P; ++p) {
            red[wave][p] = ls[p];
            red[wave][kMaxP + p] = cs[p];
            red[wave][2 * kMaxP + p] = gs[p];
        }
    __syncthreads();
    const int t = threadIdx.x;
    if (t < 3 * P) {
        const int slot = (t / P) * kMaxP + t % P;
        const float v = (red[0][slot] + red[1][slot]) + (red[2][slot] + red[3][slot]);
        a.parts[(int64_t)blockIdx.x * 3 * P + t] = v;  // [block][0: softplus(-l) | 1: sigma(-l) cos | 2: sigma(-l)][p]
    }
}

// One workgroup: fixed-order sums of the blocks' partials, folded into the outputs of the
// dense passes (loss, L^p, dL/dscale, dL/dbias).  Per listed cell and prefix the loss gains
// softplus(-l^p) / den and the residual is -sigma(-l^p) / den, which dL/ds takes times cos^p.
__global__ __launch_bounds__(256) void k_pos_fold(PosFoldArgs a) {
    __shared__ double red[256];
    __shared__ double sums[3 * kMaxP];
    const int P = a.pf.n;
    for (int t = 0; t < 3 * P; ++t) {
        double v = 0.0;
        for (int64_t b = threadIdx.x; b < a.nblk; b += 256) v += (double)a.parts[b * 3 * P + t];
        red[threadIdx.x] = v;
        __syncthreads();
        for (int h = 128; h >= 1; h >>= 1) {
            if ((int)threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
            __syncthreads();
        }
        if (threadIdx.x == 0) sums[t] = red[0];
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    double dloss = 0.0, dscale = 0.0, dbias = 0.0;
    for (int p = 0; p < P; ++p) {
        const double dl = sums[p] * a.norm;  // change of L^p
        if (a.prefix_losses_out) a.prefix_losses_out[p] = (float)((double)a.prefix_losses_out[p] + dl);
        dloss += (double)a.wnorm[p] * dl;
        dscale -= (double)a.wnorm[p] * sums[P + p] * a.norm;
        dbias -= (double)a.wnorm[p] * sums[2 * P + p] * a.norm;
    }
    *a.loss_out = (float)((double)*a.loss_out + dloss);
    if (a.dscale_out) *a.dscale_out = (float)((double)*a.dscale_out + dscale);
    if (a.dbias_out) *a.dbias_out = (float)((double)*a.dbias_out + dbias);
}

}  // namespace

hipError_t launch_pos(const PosArgs &a, hipStream_t s, int64_t *blocks_out) {
    int64_t blocks = (a.NO + 3) / 4;
    if (blocks > kPosBlocks) blocks = kPosBlocks;
    if (blocks_out) *blocks_out = blocks;
    if (a.D > 1024)
        hipLaunchKernelGGL(k_pos<2>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(k_pos<1>, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pos_fold(const PosFoldArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(k_pos_fold, dim3(1), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace uform
