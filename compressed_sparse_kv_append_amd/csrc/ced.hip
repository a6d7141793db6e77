// ced.hip -- the CED projection: the decoder's new cache entries as one
// hidden state times a projection [P2 四、"CED：上半段模型的 KV 由下半段代算"
// (the layers of the second half take their global KV from the first half's
// last output through a projection of their own)].
//
// out[r][n] = sum_k h[r][k] * w[n][k]: h bf16 [rows][d_model], w bf16
// [n_out][d_model] (one row per output channel, the contraction dimension
// contiguous in both operands), out fp32 [rows][n_out].  A true dense
// contraction, so it runs on the bf16 MFMA (v_mfma_f32_16x16x32_bf16): both
// operands are K-contiguous, so each lane's 8-element operand slice is one
// 16-byte load straight from HBM with no LDS transpose.
//
// A block owns 64 rows x 16 output channels; its 4 waves split d_model into
// quarters, each accumulating 4 row tiles against the same weight slice, and
// the 4 partial tiles are added in LDS in a fixed order (((w0 + w1) + w2) +
// w3), so results do not depend on scheduling.  At decode (rows = batch) the
// grid is n_out / 16 column blocks and the weight matrix is read once.
#include "cskv.h"
#include "device.hpp"
#include "launch.hpp"

namespace cskv {
namespace {

constexpr int kCedWaves = 4;
constexpr int kCedRows = 64;                      // rows per block (4 tiles of 16)
constexpr int kCedCols = 16;                      // output channels per block

struct CedArgs {
    const uint16_t *h;
    const uint16_t *w;
    float *out;
    int64_t rows;
    int d_model, n_out;
};

__global__ __launch_bounds__(kCedWaves * kWave) void ced_project_kernel(CedArgs a)
{
    __shared__ float part[kCedWaves][kCedRows][kCedCols];
    const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
    const int col = lane & 15, grp = lane >> 4;
    const int n0 = blockIdx.x * kCedCols;
    const int64_t r0 = (int64_t)blockIdx.y * kCedRows;
    const int kq = a.d_model / kCedWaves;         // this wave's share of the contraction
    const int kbeg = wv * kq + 8 * grp;

    // operand slices: B column = weight row n0 + col; A row = input row of tile i
    const u32x4_t *wp = reinterpret_cast<const u32x4_t *>(a.w + (size_t)(n0 + col) * a.d_model + kbeg);
    const u32x4_t *hp[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t r = r0 + 16 * i + col;
        live[i] = r < a.rows;
        hp[i] = reinterpret_cast<const u32x4_t *>(a.h + (size_t)(live[i] ? r : 0) * a.d_model + kbeg);
    }
    f32x4_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const u32x4_t zero = {0u, 0u, 0u, 0u};
#pragma unroll 4
    for (int s = 0; s < kq / 32; ++s) {           // 32 contraction slots per step = 4 u32x4 per row
        const u32x4_t b = wp[4 * s];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4_t av = live[i] ? hp[i][4 * s] : zero;
            acc[i] = mfma16x16x32(av, b, acc[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) part[wv][16 * i + 4 * grp + v][col] = acc[i][v];
    __syncthreads();
    for (int o = threadIdx.x; o < kCedRows * kCedCols; o += kCedWaves * kWave) {
        const int rr = o / kCedCols, cc = o % kCedCols;
        const int64_t r = r0 + rr;
        if (r < a.rows) {
            float s = part[0][rr][cc] + part[1][rr][cc];
            s += part[2][rr][cc];
            s += part[3][rr][cc];
            a.out[(size_t)r * a.n_out + n0 + cc] = s;
        }
    }
}

}  // namespace

hipError_t launch_ced_project(const uint16_t *h, int64_t rows, int d_model, const uint16_t *w, int n_out,
                              float *out, hipStream_t s)
{
    if (rows == 0) return hipSuccess;
    const CedArgs a{h, w, out, rows, d_model, n_out};
    const dim3 grid((unsigned)(n_out / kCedCols), (unsigned)((rows + kCedRows - 1) / kCedRows));
    launch_kernel(ced_project_kernel, grid, dim3(kCedWaves * kWave), s, nullptr, nullptr, a);
    return hipGetLastError();
}

}  // namespace cskv
