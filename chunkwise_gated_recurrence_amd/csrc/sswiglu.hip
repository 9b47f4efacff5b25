// sswiglu.hip -- GTR's Spatial SwiGLU channel mixer on gfx950 (summary page
// "GTR:门控Token循环实现高效稠密预测", section 前置知识 › SwiGLU前馈块): the
// SwiGLU mixer SiLU(X W_g) ⊙ (X W_v) W_o with a 3x3 depthwise convolution in
// the value branch,
//
//     Y = (SiLU(X W_g) ⊙ DWConv3x3(X W_v)) W_o,
//
// over the tokens of the patch grid (the convolution is a per-channel
// cross-correlation with zero padding and an optional bias). Two kernels:
//
//  * up: one workgroup per (8x8 tile of tokens, 128 hidden channels, 32 per
//    wave). It forms X W_v for the tile and its one-token halo (100 tokens, 7
//    MFMA row blocks) and X W_g for the tile (4 row blocks) on fp16 MFMA
//    16x16x32 with fp32 accumulation, the X rows and the slice's W_g / W_v
//    rows staged in LDS by buffer-to-LDS DMA through a three-stage ring
//    (kUpStages), then the convolution, the bias and the SiLU gate in fp32
//    from the accumulators (X W_v goes through LDS for the neighbours), and
//    writes the gated hidden tile A once, in fp16. X W_g and X W_v never go
//    to memory.
//  * down: Y = A W_o as a plain tiled MFMA product, 64x64 output tiles (64x32
//    when the 64x64 tiles would not cover the CUs), A and W_o staged by DMA
//    through a four-stage ring.
//
// Weights are linear-layer weights [out, in] (fp16): W_g, W_v [Hd, C],
// W_o [C, Hd]; every operand row is contiguous along the reduced dimension,
// which is the layout the MFMA operands take (16 bytes per lane).
#include "gla_common.h"
#include "gla_launch.h"

namespace gtrgla {
namespace {

typedef _Float16 sh8 __attribute__((ext_vector_type(8)));
typedef float sf4 __attribute__((ext_vector_type(4)));

constexpr int kTileSide = 8;          // core tile: 8 x 8 tokens
constexpr int kHaloTokens = 100;      // 10 x 10
constexpr int kRowBlocks = 7;         // MFMA row blocks over the halo (112 rows)
constexpr int kStageRows = 128;       // X rows staged per step (8 DMA instructions; 112..127 zero)
constexpr int kSlice = 128;           // hidden channels per workgroup, 32 per wave
constexpr int kWaveCh = kSlice / 4;
constexpr int kNB = kWaveCh / 16;     // MFMA column blocks per wave
constexpr int kUpStages = 3;          // DMA ring depth of the up kernel (two workgroups per CU)
constexpr int kStages = 4;            // DMA ring depth of the down kernel
// bytes per up-kernel stage (32 features): the X rows, then the W_g rows and
// the W_v rows of the slice's channels (64 bytes per row each)
constexpr int kUpX = kStageRows * 64;
constexpr int kUpStage = kUpX + 2 * kSlice * 64;
constexpr int kHvStride = kWaveCh + 1;             // floats per H_v row in the epilogue
constexpr int kOtStride = kSlice + 8;              // halves per row of the output tile
constexpr int kUpHvBytes = 4 * kHaloTokens * kHvStride * 4;
constexpr int kUpLds = kUpHvBytes + 64 * kOtStride * 2;   // epilogue
constexpr int kUpRing = kUpStages * kUpStage;
constexpr int kUpLdsAll = kUpLds > kUpRing ? kUpLds : kUpRing;   // the epilogue reuses the ring
// down-kernel ring stage: the A tile (64 rows) and the W_o tile (TN rows), 64
// features each
template <int TN>
constexpr int kDownStage = (64 + TN) * 128;
template <int TN>
constexpr int kDownLds = kStages * kDownStage<TN>;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_bytes(const void* p, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, unsigned char* lds, unsigned voff)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                             voff, 0, 0, 0);
}

// vmcnt(n) with the other counters left alone
template <int N>
__device__ __forceinline__ void wait_vm()
{
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Halo rows (the MFMA row order of the halo tile): the 64 core tokens first
// (row-major), then the ring: the row above and the row below (10 each, left
// to right), the column left and the column right (8 each). halo_coord gives
// (hi, hj) in [-1, 8] relative to the tile corner for row r < 100.
__device__ __forceinline__ void halo_coord(int r, int& hi, int& hj)
{
    if (r < 64) {
        hi = r >> 3;
        hj = r & 7;
    } else if (r < 74) {
        hi = -1;
        hj = r - 65;
    } else if (r < 84) {
        hi = kTileSide;
        hj = r - 75;
    } else if (r < 92) {
        hi = r - 84;
        hj = -1;
    } else {
        hi = r - 92;
        hj = kTileSide;
    }
}

// z * sigmoid(z) with the hardware reciprocal (1 ulp; the result is rounded to fp16)
__device__ __forceinline__ float silu(float z) { return z * __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Workgroup barrier for LDS: this wave's LDS accesses complete, then the
// barrier, which the compiler may not move memory accesses across. (A fence
// of workgroup scope would also wait for every DMA in flight, so that the
// ring's later stages could not overlap the current one; each ring step
// waits for its own stage with an explicit vmcnt before this barrier.)
__device__ __forceinline__ void lds_sync()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), the others unchanged
    asm volatile("s_barrier" ::: "memory");
}

}  // namespace

struct SsUpArgs {
    const _Float16* x;     // [B, L, C]
    const _Float16* wg;    // [Hd, C]
    const _Float16* wv;    // [Hd, C]
    const float* cw;       // [Hd, 3, 3]
    const float* cb;       // [Hd] or null
    _Float16* a;           // [B, L, Hd]
    int gh, gw, C, Hd;
    int tiles_w, tiles_img, slices, items, per_xcd;
};

// One workgroup per (tile, slice) work item; the items of one tile (its
// channel slices, which read the same X rows) are given consecutive block ids
// modulo 8, i.e. the same XCD and L2.
__global__ void __launch_bounds__(256) sswiglu_up_kernel(SsUpArgs p)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // A padding block (the grid is rounded up to whole XCD shares) works out
    // item 0's addresses and taps and leaves before its first DMA: the exit
    // after the argument loads lets them issue together.
    const int item_id = (int)(blockIdx.x & 7) * p.per_xcd + (int)(blockIdx.x >> 3);
    const bool live = item_id < p.items;
    const int item = live ? item_id : 0;
    const int tile = item / p.slices, slice = item - tile * p.slices;
    const int b = tile / p.tiles_img, st = tile - b * p.tiles_img;
    const int ti0 = (st / p.tiles_w) * kTileSide, tj0 = (st % p.tiles_w) * kTileSide;
    const int L = p.gh * p.gw;
    const unsigned xbytes = (unsigned)L * (unsigned)p.C * 2u;
    const __amdgpu_buffer_rsrc_t rx = rsrc_bytes(p.x + (size_t)b * L * p.C, xbytes);

    // DMA of one step (32 features = 64 bytes per row): instruction i covers
    // rows 16i .. 16i + 15, lane l row 16i + (l >> 2) into slot l & 3, which
    // holds the row's piece (l & 3) ^ ((row >> 2) & 3) (conflict-free reads).
    // Wave w issues instructions i = w and w + 4. Rows past the halo, or
    // tokens off the grid, read past the resource: zeros.
    const int n = lane & 15, kb = lane >> 4;
    const int ch0 = slice * kSlice + kWaveCh * w;   // the wave's first channel
    unsigned voff[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 16 * (w + 4 * j) + (lane >> 2);
        const int piece = (lane & 3) ^ ((row >> 2) & 3);
        unsigned v = xbytes;
        if (row < kHaloTokens) {
            int hi, hj;
            halo_coord(row, hi, hj);
            const int gi = ti0 + hi, gj = tj0 + hj;
            if (gi >= 0 && gi < p.gh && gj >= 0 && gj < p.gw)
                v = (unsigned)(gi * p.gw + gj) * (unsigned)p.C * 2u + 16u * piece;
        }
        voff[j] = v;
    }
    // The W_g and W_v rows of the wave's own channels go through the same
    // ring: kNB instructions each (rows ch0 + 16c + (l >> 2), same swizzle).
    const unsigned wbytes = (unsigned)p.Hd * (unsigned)p.C * 2u;
    const __amdgpu_buffer_rsrc_t rg = rsrc_bytes(p.wg, wbytes), rv = rsrc_bytes(p.wv, wbytes);
    const int wrow = lane >> 2, wpiece = (lane & 3) ^ ((wrow >> 2) & 3);
    const unsigned vwo = (unsigned)(ch0 + wrow) * (unsigned)p.C * 2u + 16u * wpiece;
    constexpr int kPerStage = 2 + 2 * kNB;   // DMA instructions per wave and stage
    const int nk = p.C >> 5;
    // Stage t into slot t % kUpStages; stages past nk read past the resources
    // (zeros) into slots no step reads, so that every step issues the same
    // instructions and waits for the same count.
    auto issue = [&](int t) {
        const bool in = t < nk;
        unsigned char* slot = lds + (t % kUpStages) * kUpStage;
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(rx, slot + (w + 4 * j) * 1024, in ? voff[j] + 64u * t : xbytes);
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
            const unsigned o = in ? vwo + (unsigned)(16 * c) * (unsigned)p.C * 2u + 64u * t : wbytes;
            dma16(rg, slot + kUpX + (kNB * w + c) * 1024, o);
            dma16(rv, slot + kUpX + (4 * kNB + kNB * w + c) * 1024, o);
        }
    };

    // the lane's convolution taps and bias for each of its channels (used after the loop)
    float tap[kNB][9], bias[kNB];
#pragma unroll
    for (int c = 0; c < kNB; ++c) {
        const int ch = ch0 + 16 * c + n;
#pragma unroll
        for (int t = 0; t < 9; ++t) tap[c][t] = p.cw[(size_t)ch * 9 + t];
        bias[c] = p.cb ? p.cb[ch] : 0.f;
    }

    if (!live) return;

    sf4 accv[kRowBlocks][kNB], accg[4][kNB];
#pragma unroll
    for (int i = 0; i < kRowBlocks; ++i)
#pragma unroll
        for (int c = 0; c < kNB; ++c) accv[i][c] = sf4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < kNB; ++c) accg[i][c] = sf4{0.f, 0.f, 0.f, 0.f};

    // the fragments of a 16-row block: row n, piece kb
    const int frag = n * 64 + 16 * (kb ^ ((n >> 2) & 3));
#pragma unroll
    for (int t = 0; t < kUpStages - 1; ++t) issue(t);
    for (int s = 0; s < nk; ++s) {
        // stage s has landed once only the kUpStages - 2 later stages are in flight
        wait_vm<kPerStage * (kUpStages - 2)>();
        lds_sync();
        issue(s + kUpStages - 1);   // into the slot read at s - 1
        const unsigned char* slot = lds + (s % kUpStages) * kUpStage;
        sh8 a[kRowBlocks], bg[kNB], bv[kNB];
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
            bg[c] = *reinterpret_cast<const sh8*>(slot + kUpX + (kNB * w + c) * 1024 + frag);
            bv[c] = *reinterpret_cast<const sh8*>(slot + kUpX + (4 * kNB + kNB * w + c) * 1024 + frag);
        }
#pragma unroll
        for (int i = 0; i < kRowBlocks; ++i) a[i] = *reinterpret_cast<const sh8*>(slot + i * 1024 + frag);
#pragma unroll
        for (int i = 0; i < kRowBlocks; ++i)
#pragma unroll
            for (int c = 0; c < kNB; ++c) {
                accv[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bv[c], accv[i][c], 0, 0, 0);
                if (i < 4)
                    accg[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i], bg[c], accg[i][c], 0, 0, 0);
            }
    }
    wait_vm<0>();   // the stages issued past the end land before the LDS is reused
    lds_sync();   // every wave is done with the ring

    // X W_v of the wave's channels to LDS as the 10 x 10 halo grid (position
    // (hi + 1) * 10 + hj + 1), so that the neighbours are at fixed offsets
    float* hv = reinterpret_cast<float*>(lds) + w * kHaloTokens * kHvStride;
#pragma unroll
    for (int i = 0; i < kRowBlocks; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * i + 4 * kb + e;
            if (row < kHaloTokens) {
                int hi, hj;
                halo_coord(row, hi, hj);
                float* d = hv + ((hi + 1) * 10 + hj + 1) * kHvStride + n;
#pragma unroll
                for (int c = 0; c < kNB; ++c) d[16 * c] = accv[i][c][e];
            }
        }
    lds_sync();
    // The lane's core tokens of row block i are four neighbours in one row:
    // (hi, hj0 + e) with hi = 2i + (kb >> 1), hj0 = 4 (kb & 1); their 3 x 3
    // windows lie in the 3 x 6 block of the grid at (hi, hj0).
    _Float16* ot = reinterpret_cast<_Float16*>(lds + kUpHvBytes);   // [64][kOtStride]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hi = 2 * i + (kb >> 1), hj0 = 4 * (kb & 1);
        const float* wbase = hv + (hi * 10 + hj0) * kHvStride + n;
#pragma unroll
        for (int c = 0; c < kNB; ++c) {
            float win[3][6];
#pragma unroll
            for (int a = 0; a < 3; ++a)
#pragma unroll
                for (int bb = 0; bb < 6; ++bb) win[a][bb] = wbase[(10 * a + bb) * kHvStride + 16 * c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float conv = bias[c];
#pragma unroll
                for (int a = 0; a < 3; ++a)
#pragma unroll
                    for (int bb = 0; bb < 3; ++bb) conv += tap[c][3 * a + bb] * win[a][e + bb];
                ot[(16 * i + 4 * kb + e) * kOtStride + kWaveCh * w + 16 * c + n] =
                    (_Float16)(silu(accg[i][c][e]) * conv);
            }
        }
    }
    lds_sync();
    // 64 tokens x kSlice channels, 16 bytes per thread and piece
    const size_t abase = (size_t)b * L;
    constexpr int kParts = kSlice / 8;
#pragma unroll
    for (int j = 0; j < 64 * kParts / 256; ++j) {
        const int q = tid + 256 * j;
        const int r = q / kParts, part = q % kParts;
        const int gi = ti0 + (r >> 3), gj = tj0 + (r & 7);
        if (gi < p.gh && gj < p.gw) {
            const sh8 v = *reinterpret_cast<const sh8*>(ot + r * kOtStride + 8 * part);
            *reinterpret_cast<sh8*>(p.a + (abase + gi * p.gw + gj) * p.Hd + slice * kSlice + 8 * part) = v;
        }
    }
}

struct SsDownArgs {
    const _Float16* a;     // [M, Hd]
    const _Float16* wo;    // [C, Hd]
    _Float16* y;           // [M, C]
    int M, Hd, C;
    int n_tiles, items, per_xcd;
};

// 64 x TN tiles of Y (TN = 64 or 32); wave (wm, wn) computes rows 32wm .. +31
// and columns (TN / 2) wn .. + TN / 2 - 1. A stage holds 64 features of the
// A rows and of the W_o rows (128 bytes per row; DMA instruction i covers
// rows 8i .. 8i + 7, lane l row 8i + (l >> 3) into slot l & 7, holding piece
// (l & 7) ^ ((row >> 1) & 7)). Narrow tiles double the workgroups of a small
// product, so that every CU takes part.
template <int TN>
__global__ void __launch_bounds__(256) sswiglu_down_kernel(SsDownArgs p)
{
    constexpr int NJ = TN / 32;             // 16-column blocks per wave
    constexpr int NW = TN / 32;             // W_o DMA instructions per wave and stage
    constexpr int kPer = 2 + NW;            // DMA instructions per wave and stage
    constexpr int kStage = kDownStage<TN>;
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int item = (int)(blockIdx.x & 7) * p.per_xcd + (int)(blockIdx.x >> 3);
    if (item >= p.items) return;
    const int mt = item / p.n_tiles, nt = item - mt * p.n_tiles;
    const int m0 = mt * 64, n0 = nt * TN;
    const unsigned abytes = (unsigned)p.M * (unsigned)p.Hd * 2u;
    const __amdgpu_buffer_rsrc_t ra = rsrc_bytes(p.a, abytes);
    const __amdgpu_buffer_rsrc_t rw = rsrc_bytes(p.wo, (unsigned)p.C * (unsigned)p.Hd * 2u);
    // wave w issues A instructions 2w, 2w + 1 and W_o instructions NW w .. NW w + NW - 1
    unsigned va[2], vw[NW];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int row = 8 * (2 * w + j) + (lane >> 3);
        const int piece = (lane & 7) ^ ((row >> 1) & 7);
        va[j] = m0 + row < p.M ? (unsigned)(m0 + row) * (unsigned)p.Hd * 2u + 16u * piece : abytes;
    }
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        const int row = 8 * (NW * w + j) + (lane >> 3);
        const int piece = (lane & 7) ^ ((row >> 1) & 7);
        vw[j] = (unsigned)(n0 + row) * (unsigned)p.Hd * 2u + 16u * piece;
    }
    auto issue = [&](int s) {
        unsigned char* slot = lds + (s % kStages) * kStage;
#pragma unroll
        for (int j = 0; j < 2; ++j) dma16(ra, slot + (2 * w + j) * 1024, va[j] + 128u * s);
#pragma unroll
        for (int j = 0; j < NW; ++j) dma16(rw, slot + 8192 + (NW * w + j) * 1024, vw[j] + 128u * s);
    };
    const int wm = w >> 1, wn = w & 1;
    const int n = lane & 15, kb = lane >> 4;
    sf4 acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = sf4{0.f, 0.f, 0.f, 0.f};
    const int nk = p.Hd >> 6;
    for (int s = 0; s < kStages - 1 && s < nk; ++s) issue(s);
    for (int s = 0; s < nk; ++s) {
        const int after = nk - 1 - s;
        if (after >= kStages - 2) wait_vm<kPer * (kStages - 2)>();
        else if (after == 1) wait_vm<kPer>();
        else wait_vm<0>();
        lds_sync();
        if (s + kStages - 1 < nk) issue(s + kStages - 1);
        const unsigned char* slot = lds + (s % kStages) * kStage;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const int piece = 4 * ks + kb;
            sh8 fa[2], fw[NJ];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int ra_ = 32 * wm + 16 * i + n;
                fa[i] = *reinterpret_cast<const sh8*>(slot + ra_ * 128 + 16 * (piece ^ ((ra_ >> 1) & 7)));
            }
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int rw_ = (TN / 2) * wn + 16 * j + n;
                fw[j] = *reinterpret_cast<const sh8*>(slot + 8192 + rw_ * 128 +
                                                      16 * (piece ^ ((rw_ >> 1) & 7)));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fw[j], acc[i][j], 0, 0, 0);
        }
    }
    // lane (n, kb) holds Y[row 32wm + 16i + 4kb + e][col (TN / 2) wn + 16j + n]
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = m0 + 32 * wm + 16 * i + 4 * kb + e;
            if (row < p.M) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    p.y[(size_t)row * p.C + n0 + (TN / 2) * wn + 16 * j + n] = (_Float16)acc[i][j][e];
            }
        }
}

static int per_xcd(int items) { return (items + 7) / 8; }

static int cu_count()
{
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus < 1)
            cus = 256;
        cached = cus;
    }
    return cached;
}

hipError_t launch_sswiglu(const void* x, const void* wg, const void* wv, const float* cw,
                          const float* cb, const void* wo, int B, int gh, int gw, int C, int Hd,
                          void* y, void* a_ws, hipStream_t st)
{
    static bool attrs = false;
    if (!attrs) {
        if (hipFuncSetAttribute((const void*)sswiglu_up_kernel,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kUpLdsAll) != hipSuccess ||
            hipFuncSetAttribute((const void*)sswiglu_down_kernel<64>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kDownLds<64>) != hipSuccess ||
            hipFuncSetAttribute((const void*)sswiglu_down_kernel<32>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, kDownLds<32>) != hipSuccess)
            return hipGetLastError();
        attrs = true;
    }
    SsUpArgs u;
    u.x = (const _Float16*)x;
    u.wg = (const _Float16*)wg;
    u.wv = (const _Float16*)wv;
    u.cw = cw;
    u.cb = cb;
    u.a = (_Float16*)a_ws;
    u.gh = gh;
    u.gw = gw;
    u.C = C;
    u.Hd = Hd;
    u.tiles_w = (gw + kTileSide - 1) / kTileSide;
    u.tiles_img = u.tiles_w * ((gh + kTileSide - 1) / kTileSide);
    u.slices = Hd / kSlice;
    u.items = B * u.tiles_img * u.slices;
    u.per_xcd = per_xcd(u.items);
    hipLaunchKernelGGL(sswiglu_up_kernel, dim3(8 * u.per_xcd), dim3(256), kUpLdsAll, st, u);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    SsDownArgs d;
    d.a = (const _Float16*)a_ws;
    d.wo = (const _Float16*)wo;
    d.y = (_Float16*)y;
    d.M = B * gh * gw;
    d.Hd = Hd;
    d.C = C;
    // 64-column tiles; 32-column ones when the 64-column tiles would leave CUs idle
    const bool narrow = ((d.M + 63) / 64) * (C / 64) < cu_count();
    d.n_tiles = narrow ? C / 32 : C / 64;
    d.items = ((d.M + 63) / 64) * d.n_tiles;
    d.per_xcd = per_xcd(d.items);
    if (narrow)
        hipLaunchKernelGGL(sswiglu_down_kernel<32>, dim3(8 * d.per_xcd), dim3(256), kDownLds<32>, st, d);
    else
        hipLaunchKernelGGL(sswiglu_down_kernel<64>, dim3(8 * d.per_xcd), dim3(256), kDownLds<64>, st, d);
    return hipGetLastError();
}

}  // namespace gtrgla
