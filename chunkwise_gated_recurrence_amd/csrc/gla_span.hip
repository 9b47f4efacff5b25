// gla_span.hip -- the span kernels: the fused fp16 path of libgtrgla for
// d_v = 64, d_k in {32, 64}, chunk C = 64, on gfx950 (CDNA4) MFMA.
//
// It evaluates the chunkwise form of key-only GLA (GTR summary page
// "GTR:门控Token循环实现高效稠密预测", section 前置知识 › Chunkwise(分块)并行 and
// the operator of section 方法步骤详情; 0539edu.com page, section 3.3): chunk
// summaries U_c and decays d_c, the boundary scan S_[c+1] = Diag(d_c) S_[c] +
// U_c, and per-chunk outputs, in one launch.
//
// Work decomposition. Each (batch, head) sequence is cut into n_spans spans of
// SPAN consecutive 64-token chunks, one workgroup of four waves per span, and
// every workgroup of a launch is resident at once (the host sizes spans and
// sequence batches from the measured occupancy).
//   1. Local pass over the span's chunks from a zero state: intra-chunk
//      outputs plus the contribution of the span-local state, kept on chip
//      (fp16, registers) with the operand q 2^{b+P} that the incoming state
//      will multiply; the state in registers.
//   2. Boundary exchange between the span workgroups of a sequence: each span
//      publishes its summary as tagged words; owners fold a slice of every
//      span's summary on registers and write each span's incoming state; every
//      span polls its own (state elements travel in row-quad order, so that
//      each lane moves whole 16- and 8-byte pieces).
//   3. Outputs: kept outputs plus (q 2^{b+P}) S_in, stored at the spatial rows.
//
// Per chunk, wave w owns tokens 16w .. 16w+15 (scores and outputs) and value
// columns 16w .. 16w+15 of the state (state rows i are the key dims). MFMA
// 16x16x32 fp16 -> fp32 throughout. With lane l = (n = l & 15, g = l >> 4):
//   * "b-layout": lane (n, g) of wave w holds, for token t = 16w + n, the key
//     dims 16 db + 4 g + e (db = 0 .. d_k/16 - 1, e = 0 .. 3). q and k are
//     read into it from their staged tiles (8-byte pieces); the log-gate
//     prefix lands in it.
//   * The log-gate prefix b_t = sum_{s <= t} log gamma_s is an MFMA of the
//     staged gate tile (read transposed from LDS) against a 0/1 lower-triangle
//     operand, and the chunk total against ones, so every wave has every
//     per-dim quantity of its dims without any exchange between waves.
//   * Scores use (q 2^{b-r}) (k 2^{r-b})^T with r = b_last / 2 (every factor in
//     [2^-8, 2^8] while the chunk's log2 decay is at most 16 per dim); a chunk
//     with a stronger decay takes its scores exactly in fp32 instead (a walk
//     over the keys with the running decay).
//   * g, v, q and k are staged by buffer-to-LDS DMA one chunk ahead; operands
//     that need a tile transposed (v^T, (k 2^{r-b})^T, the gate tile) are read
//     with the LDS transpose read (ds_read_b64_tr_b16). 16-byte pieces of every
//     tile row are XOR-swizzled by the row index.
//   * The contraction index of every product is permuted consistently on both
//     operands, so that an MFMA result feeds the next MFMA straight from its
//     accumulator registers (scores into scores x V; the state into q S).
// Two barriers per chunk: after the staged data has landed (and the previous
// chunk's tiles are free), and after the k 2^{r-b} and state tiles are written.
#include <cstdlib>

#include "gla_common.h"
#include "gla_launch.h"
#include "gla_ws.h"

namespace gtrgla {
namespace span {

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u2 __attribute__((ext_vector_type(2)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;             // chunk length
constexpr int kDV = 64;            // value dim
constexpr int kThreads = 256;      // four waves
constexpr int kMaxSpan = 7;        // longest span kept on chip
constexpr int kMaxSpans = 64;      // spans per sequence
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGuard = 16.0f;    // largest log2 decay of a chunk for the factorised scores
constexpr int kDevScope = 16;      // cache policy: device-scope (sc1) access
constexpr int kPollSleep = 2;      // s_sleep between incoming-state polls

// ---------------------------------------------------------------------------
// small helpers

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// Barrier that orders LDS only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Scheduling fence: no instruction moves across it, which bounds how many
// operand loads the scheduler hoists (and keeps live) ahead of their MFMAs.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

__device__ __forceinline__ h8 cat(h4 a, h4 b) { return h8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }
__device__ __forceinline__ h4 lo4(h8 a) { return h4{a[0], a[1], a[2], a[3]}; }
__device__ __forceinline__ h4 hi4(h8 a) { return h4{a[4], a[5], a[6], a[7]}; }
__device__ __forceinline__ h4 cvt4(f4 x) { return h4{(_Float16)x[0], (_Float16)x[1], (_Float16)x[2], (_Float16)x[3]}; }
__device__ __forceinline__ f4 up4(h4 x) { return f4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }

// Buffer resource over n_bytes at base: accesses past the end read zeros and
// are dropped on write.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int n_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n_bytes, 0x00020000);
}

// Element offset (halves) of column `col` (a multiple of 4) of row `row` in an
// LDS tile of R halves per row whose 16-byte pieces are XOR-swizzled by the row.
template <int R>
__device__ __forceinline__ int sw(int row, int col)
{
    constexpr int P = R / 8;   // pieces per row
    return row * R + ((((col >> 3) ^ row) & (P - 1)) << 3) + (col & 7);
}

typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 tr_h4;
// Transposed 16x4 read: lane (m, kb) of the wave receives rows row0 + 4 kb + e
// (e = 0 .. 3) of column col0 + m of the tile (the hardware gathers the 8-byte
// pieces that lanes 4e + q of each 16-lane group address: row row0 + 4 kb + e,
// columns col0 + 4q .. + 3).
//
// Addresses of the accesses below split in two: with the row a multiple of 16
// plus a lane part and the column a multiple of 16 (32 for 8-wide pieces) plus
// a lane part, the swizzled piece ((col >> 3) ^ row) & (P - 1) is the block's
// bits (col & (R - 8)) XOR the lane's, so the lane's terms are computed once
// per chunk and an access adds only its block's (no carries: the block's
// column bits and the lane's column bits do not overlap).
template <int R>
__device__ __forceinline__ h4 tr_read(const _Float16* tile, int row0, int col0, int lane)
{
    constexpr int P = R / 8;
    const int rl = 4 * (lane >> 4) + ((lane & 15) >> 2);   // row within the block
    const int x8 = ((((lane >> 1) & 1) ^ rl) & (P - 1)) << 3;
    const int off = row0 * R + rl * R + 4 * (lane & 1) + ((col0 & (R - 8)) ^ x8);
    auto p = (__attribute__((address_space(3))) tr_h4*)(
        (__attribute__((address_space(3))) _Float16*)(tile + off));
    return __builtin_bit_cast(h4, __builtin_amdgcn_ds_read_tr16_b64_v4f16(p));
}
// Row rb + n, columns c + 4g .. + 3 (lane (n, g); rb and c multiples of 16).
template <int R>
__device__ __forceinline__ int off4g(int rb, int c, int lane)
{
    constexpr int P = R / 8;
    const int n = lane & 15, g = lane >> 4;
    return (rb + n) * R + 4 * (g & 1) + ((c & (R - 8)) ^ ((((g >> 1) ^ n) & (P - 1)) << 3));
}
// Row rb + n, columns c + 8g .. + 7 (rb a multiple of 16, c of 32).
template <int R>
__device__ __forceinline__ int off8g(int rb, int c, int lane)
{
    constexpr int P = R / 8;
    const int n = lane & 15, g = lane >> 4;
    return (rb + n) * R + ((c & (R - 8)) ^ (((g ^ n) & (P - 1)) << 3));
}
// The two transposed reads of one 32-deep contraction step in the permuted
// order used throughout: lane (m, kb), element e' < 4: row 32 ks + 4 kb + e';
// e' >= 4: row 32 ks + 16 + 4 kb + e' - 4.
template <int R>
__device__ __forceinline__ h8 tr_step(const _Float16* tile, int ks, int col0, int lane)
{
    return cat(tr_read<R>(tile, 32 * ks, col0, lane), tr_read<R>(tile, 32 * ks + 16, col0, lane));
}
template <int R>
__device__ __forceinline__ h4 ld4(const _Float16* tile, int row, int col)
{
    return *reinterpret_cast<const h4*>(tile + sw<R>(row, col));
}
template <int R>
__device__ __forceinline__ h4 ld4g(const _Float16* tile, int rb, int c, int lane)
{
    return *reinterpret_cast<const h4*>(tile + off4g<R>(rb, c, lane));
}
template <int R>
__device__ __forceinline__ void st4g(_Float16* tile, int rb, int c, int lane, h4 x)
{
    *reinterpret_cast<h4*>(tile + off4g<R>(rb, c, lane)) = x;
}
template <int R>
__device__ __forceinline__ h8 ld8g(const _Float16* tile, int rb, int c, int lane)
{
    return *reinterpret_cast<const h8*>(tile + off8g<R>(rb, c, lane));
}
template <int R>
__device__ __forceinline__ void st8g(_Float16* tile, int rb, int c, int lane, h8 x)
{
    *reinterpret_cast<h8*>(tile + off8g<R>(rb, c, lane)) = x;
}

// Tagged exchange words: summaries are fp32 rounded to nearest at 16 mantissa
// bits with an 8-bit tag in the low bits; incoming states are fp16 whose
// lowest mantissa bit carries the tag's parity (the output pass multiplies
// them in fp16; every launch that uses a slot rewrites all of its words and
// advances its epoch by one, so a stale word carries the previous parity).
__device__ __forceinline__ unsigned int ll_word(float v, unsigned int tag)
{
    return ((__float_as_uint(v) + 0x80u) & 0xFFFFFF00u) | tag;
}
__device__ __forceinline__ float ll_value(unsigned int x) { return __uint_as_float(x & 0xFFFFFF00u); }
__device__ __forceinline__ bool ll_ok(unsigned int x, unsigned int tag) { return (x & 0xFFu) == tag; }
__device__ __forceinline__ unsigned short sin_word(float v, unsigned int tag)
{
    const unsigned short x = __builtin_bit_cast(unsigned short, (_Float16)v);
    return (unsigned short)((x & 0xFFFEu) | (tag & 1u));
}
__device__ __forceinline__ bool sin_ok(unsigned short x, unsigned int tag) { return ((x ^ tag) & 1u) == 0; }
__device__ __forceinline__ _Float16 sin_value(unsigned short x)
{
    return __builtin_bit_cast(_Float16, (unsigned short)(x & 0xFFFEu));
}

__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

// ---------------------------------------------------------------------------
struct SpanArgs {
    const __half* q;
    const __half* k;
    const __half* v;
    const __half* lg;
    __half* out;
    float* final_state;
    unsigned int* hdr;          // workspace header (gla_ws.h)
    unsigned int* epoch;        // [seq in launch][n_spans]: tag of the slot's words (low 8 bits)
    unsigned int* agg;          // [seq in launch][agg_words]: published summaries, owner-major
    unsigned char* sin;         // [seq in launch][n_spans] slots of 2 NE bytes: incoming states
    int L, H, grid_h, grid_w, dir;
    int n_chunks;               // per sequence
    int n_spans;                // workgroups per sequence
    int seq0;                   // first sequence of this launch
    int slice_log2;             // log2 of the state elements each owner folds
    int agg_words;              // summary words per sequence
    float scale;                // d_k^{-1/2}
    float inv_gh;               // 1 / grid_h
    const float* init;          // [B, H, d_k, 64] state before the first step, or null
    const __half* gate;         // [B, L, H, 64] output gate, or null
    const float* norm_w;        // [64] RMSNorm weight (with gate)
    float eps;
    unsigned int layout;        // exchange layout word (header word 2)
    int fault;                  // test hook: span 0 of every sequence publishes nothing
    unsigned long long wait_ticks;   // longest wait of one poll loop (wall-clock ticks)
};

// LDS of one workgroup. A stage holds one chunk's g, v, q and k tiles (rows =
// tokens in scan order), staged by DMA one chunk ahead (two stages when the
// span has two or more chunks). Within a chunk each wave reads only its own
// rows of q and k, then overwrites them: its rows of the q tile with its
// columns of the state operand T[j][permuted i], its rows of the k tile with
// k 2^{a t - b}. After the local pass: the exchange's scratch (the fold's
// range aggregates, at the start of the stage region) and the incoming state
// (the last kTin bytes).
template <int DK, int NS>
struct Lds {
    struct Stage {
        _Float16 g[kC * DK];    // log gates
        _Float16 v[kC * kDV];
        _Float16 q[kC * DK];    // q; then T
        _Float16 k[kC * DK];    // k; then k 2^{r-b} (or k 2^{b_last-b})
    } stage[NS];
    unsigned int tags[kMaxSpans];   // expected tag of every span slot of the sequence
    unsigned int hdr[4];        // the workspace header, staged at the start
    // the owners' poll rounds: per-wave "a word was stale" and the deadline,
    // double-buffered by round parity (one barrier per round)
    int stale_w[2][4], expired_r[2];
    int poison;

    static constexpr int kTin = kDV * DK * 2;   // incoming state, fp16 [j][permuted i]
    __device__ unsigned char* region() { return reinterpret_cast<unsigned char*>(&stage[0]); }
    static constexpr int kRegion = (int)(sizeof(Stage) * NS);
    __device__ _Float16* tin() { return reinterpret_cast<_Float16*>(region() + kRegion - kTin); }
    static constexpr int kScratch = kRegion - kTin;
    static_assert(kScratch >= 256 * 4, "the fold's decays fit below the incoming state");
};

// ---------------------------------------------------------------------------
// loads

// Scan order -> spatial position for the rows of one chunk. The scan orders
// l2r / r2l walk the grid row-major (forwards / backwards), t2b / b2t
// column-major. The uniform part (for the column-major orders: the column and
// row of the chunk's first step) is computed once per chunk; a lane's row then
// takes a few VALU operations and no integer division: with x the row offset
// from the chunk start's row, floor((x + 1/2) / grid_h) is exact in fp32, as
// (x + 1/2) / grid_h stays 1 / (2 grid_h) away from every integer, far more
// than the rounding error for |x| < grid_h + 64.
struct RowMap {
    int t0;       // first scan step of the chunk
    int c0, r0;   // column-major orders: column and row of t0's scan position
};
__device__ __forceinline__ RowMap row_map(const SpanArgs& a, int t0)
{
    RowMap m;
    m.t0 = t0;
    m.c0 = m.r0 = 0;
    if (a.dir >= 2) {   // uniform
        const int u0 = a.dir == 3 ? a.L - 1 - t0 : t0;
        m.c0 = u0 / a.grid_h;
        m.r0 = u0 - m.c0 * a.grid_h;
    }
    return m;
}
// spatial position of scan step t0 + r (0 <= r < 64), or -1 past the sequence end
__device__ __forceinline__ int row_pos(const SpanArgs& a, const RowMap& m, int r)
{
    const int t = m.t0 + r;
    int p;
    if (a.dir >= 2) {
        const int x = a.dir == 3 ? m.r0 - r : m.r0 + r;
        const int q = (int)__builtin_floorf(((float)x + 0.5f) * a.inv_gh);
        p = (x - q * a.grid_h) * a.grid_w + m.c0 + q;
    } else {
        p = a.dir == 1 ? a.L - 1 - t : t;
    }
    return t < a.L ? p : -1;
}
// byte offset of spatial position p of head h in a [B, L, H, R] fp16 tensor,
// relative to batch b; -1 (past the end): `end` (reads zeros)
template <int R>
__device__ __forceinline__ int pos_bytes(const SpanArgs& a, int h, int p, int end)
{
    return p < 0 ? end : (p * a.H + h) * (R * 2);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t batch_rsrc(const __half* base, const SpanArgs& a,
                                                             int b, int R)
{
    const long long per_batch = (long long)a.L * a.H * R;
    return rsrc(base + b * per_batch, (int)(per_batch * 2));
}

// Stage the chunk's g, v, q and k tiles into an LDS stage by buffer-to-LDS DMA.
// A DMA instruction writes 64 consecutive 16-byte pieces; lane l fetches the
// piece of its row that the row's XOR swizzle puts at LDS position l. Each wave
// stages rows 16w .. 16w + 15: a 64-wide tile in two instructions (rows
// 16w + 8i + l / 8), a 32-wide one in one (rows 16w + l / 4); the rows'
// positions are shared by the tiles of one width.
template <int R>
__device__ __forceinline__ void dma_tile(const SpanArgs& a, __amdgpu_buffer_rsrc_t rs, _Float16* tile,
                                         int h, const int* pos, int w, int lane)
{
    constexpr int P = R / 8;           // pieces per row
    constexpr int RPI = 64 / P;        // rows per DMA instruction
    const int end = a.L * a.H * R * 2;
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
        const int row = 16 * w + RPI * i + lane / P;
        const int piece = (lane % P) ^ (row & (P - 1));
        const int off = pos_bytes<R>(a, h, pos[i], end);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (__attribute__((address_space(3))) void*)(tile + (16 * w + RPI * i) * R), 16,
            off == end ? end : off + 16 * piece, 0, 0, 0);
    }
}
template <class St>
__device__ __forceinline__ void dma_stage(const SpanArgs& a, St& st, int b, int h, int t0, int w,
                                          int lane)
{
    constexpr int DK = sizeof(st.q) / (2 * kC);
    const RowMap m = row_map(a, t0);
    const int p64[2] = {row_pos(a, m, 16 * w + (lane >> 3)), row_pos(a, m, 16 * w + 8 + (lane >> 3))};
    const int p32[1] = {DK == 32 ? row_pos(a, m, 16 * w + (lane >> 2)) : 0};
    const int* pk = DK == 32 ? p32 : p64;
    dma_tile<DK>(a, batch_rsrc(a.lg, a, b, DK), st.g, h, pk, w, lane);
    dma_tile<kDV>(a, batch_rsrc(a.v, a, b, kDV), st.v, h, p64, w, lane);
    dma_tile<DK>(a, batch_rsrc(a.q, a, b, DK), st.q, h, pk, w, lane);
    dma_tile<DK>(a, batch_rsrc(a.k, a, b, DK), st.k, h, pk, w, lane);
}

// ---------------------------------------------------------------------------
// One chunk of the local pass.

// 0/1 operand of the gate prefix: tri (lane (n, kb) of wave w, element e':
// token s = 32 ks + 16 (e' >= 4) + 4 kb + (e' & 3) <= t = 16 w + n). Built
// where it is used (a few VALU operations) rather than held across chunks.
__device__ __forceinline__ h8 tri_operand(int w, int lane, int ks)
{
    const int t = 16 * w + (lane & 15), kb = lane >> 4;
    h8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        r[e] = (32 * ks + 16 * (e >> 2) + 4 * kb + (e & 3) <= t) ? (_Float16)1.f : (_Float16)0.f;
    return r;
}

// What a chunk leaves for the span's output pass: intra-chunk plus span-local
// outputs (fp16; O^T layout: lane (n, g) of wave w holds token 16w + n,
// columns 16 jt + 4 g .. + 3) and Qs = q 2^{b} D_c in the permuted dim order
// (D_c: decay from the span start to the chunk start).
template <int DK>
struct Kept {
    h4 o[4];
    h8 qs[DK / 32];
};

template <int DK>
struct ChunkState {
    f4 S[DK / 16];      // state (rows i = 16 it + 4 g + e, column 16 w + n)
    h4 Dp[DK / 16];     // decay from the span start (dims 16 db + 4 g + e), fp16: it
                        // only scales the kept q operand (a tiny value may underflow,
                        // as its contribution does)
};

// The chunk's gates: inclusive prefix b (b-layout) and total b_last, both as
// natural logs, from the staged gate tile.
template <int DK>
__device__ __forceinline__ void chunk_gates(const _Float16* G, int w, int lane, int lane_tri,
                                            f4 (&bsum)[DK / 16], f4 (&tot)[DK / 16])
{
    constexpr int NDB = DK / 16;
    const h8 ones = {(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f,
                     (_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        bsum[db] = f4{0.f, 0.f, 0.f, 0.f};
        tot[db] = f4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        const h8 tri = tri_operand(w, lane_tri, ks);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const h8 A = tr_step<DK>(G, ks, 16 * db, lane);   // G^T: dims x tokens
            tot[db] = mfma(A, ones, tot[db]);
            if (ks == 0 || w >= 2) bsum[db] = mfma(A, tri, bsum[db]);
        }
    }
}

// One chunk of the local pass. On entry cs.S is the span-local state at the
// chunk start; on exit the state after it.
//
// With t = b_last (per dim, log2 units) and a = 1/2 (factorised chunk: every
// dim's log2 decay <= kGuard) or a = 1 (wide chunk, where 2^{+-t/2} could
// overflow fp16), and a' = 1 - a:
//   q operand   q 2^{b - a' t}        k operand   k 2^{a t - b}
//   state operand of the outputs      S 2^{a' t}
//   state update                      S <- 2^{a' t} (2^{a t} S + (k operand)^T V)
// which is d_c S + (k 2^{t - b})^T V either way. Factorised, the scores are
// (q operand)(k operand)^T on MFMA; wide, the operands are at most the raw
// values and the scores are computed exactly in fp32 (q_t k_s 2^{b_t - b_s}
// summed over the dims), walking the keys down from each token with the
// running weight.
template <int DK, bool KEEPF, bool EARLY, class St, class AfterState>
__device__ __forceinline__ void chunk_step(St& st, int w, int lane, const f4 (&bsum)[DK / 16],
                                           const f4 (&tot)[DK / 16], bool wide,
                                           ChunkState<DK>& cs, Kept<DK>& kept,
                                           AfterState after_state)
{
    constexpr int NDB = DK / 16, NKS = DK / 32;
    const int n = lane & 15, g = lane >> 4;
    const int row = 16 * w + n;
    const float al = (wide ? 1.f : 0.5f) * kLog2e;   // a, with the natural-log gates
    const float be = (wide ? 0.f : 0.5f) * kLog2e;   // a'
    // q and k operands (the wave's own rows, b-layout)
    h4 qh[NDB], kh[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        f4 fq, fk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float b2 = bsum[db][e] * kLog2e;
            fq[e] = ex2(__builtin_fmaf(tot[db][e], -be, b2));
            fk[e] = ex2(__builtin_fmaf(tot[db][e], al, -b2));
        }
        qh[db] = ld4g<DK>(st.q, 16 * w, 16 * db, lane) * cvt4(fq);
        kh[db] = ld4g<DK>(st.k, 16 * w, 16 * db, lane) * cvt4(fk);
    }
    h8 qk[NKS];   // the q operand of the scores and of the state term
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qk[ks] = cat(qh[2 * ks], qh[2 * ks + 1]);
    // kept operand of the incoming state: q 2^b D_c; then D_{c+1} = D_c d_c;
    // the state operand of the outputs S 2^{a' t} (written to T once the q rows
    // are free) and the update's first term S 2^{a t}
    // (2^{a' t} is 2^{a t} for a factorised chunk, 1 for a wide one)
    f4 Tp[NDB], Sp[NDB], fbk[NDB];
#pragma unroll
    for (int it = 0; it < NDB; ++it) {
        f4 fa, fb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            fa[e] = ex2(al * tot[it][e]);
            fb[e] = KEEPF ? (wide ? 1.f : fa[e]) : ex2(be * tot[it][e]);
        }
        if (KEEPF) fbk[it] = fb;
        const f4 dp = up4(cs.Dp[it]);
        Tp[it] = cs.S[it] * fb;
        Sp[it] = cs.S[it] * fa;
        qh[it] = qh[it] * cvt4(fb * dp);
        cs.Dp[it] = cvt4(dp * fa * fb);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) kept.qs[ks] = cat(qh[2 * ks], qh[2 * ks + 1]);

    f4 sc[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) sc[sb] = f4{0.f, 0.f, 0.f, 0.f};
    if (wide) {
        // walk the keys down from the wave's last token, one block of 16 dims
        // at a time: lane (n, g) holds E[i] = 2^{b_t[i] - b_s[i]} for its token
        // t and 4 dims of the block, starting at 1 when s reaches t and
        // multiplied by gamma_{s+1} at each step down (a strong decay
        // underflows towards 0, as the true weight does)
#pragma unroll 1
        for (int db = 0; db < NDB; ++db) {
            const f4 qq = up4(ld4g<DK>(st.q, 16 * w, 16 * db, lane));
            f4 E = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int s = 16 * w + 15; s >= 0; --s) {
                const f4 gn = up4(ld4<DK>(st.g, s + 1 < kC ? s + 1 : s, 16 * db + 4 * g));
                const f4 kk = up4(ld4<DK>(st.k, s, 16 * db + 4 * g));
                float part = 0.f;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    E[e] = s > row ? 0.f : (s == row ? 1.f : E[e] * ex2(gn[e] * kLog2e));
                    part += qq[e] * kk[e] * E[e];
                }
                part += __shfl_xor(part, 16, 64);
                part += __shfl_xor(part, 32, 64);
                // lane (n, g) keeps keys 16 sb + 4 g + e; s is wave-uniform
                const int sb = s >> 4, e = s & 3;
                if (((s >> 2) & 3) == g) {
#pragma unroll
                    for (int kq = 0; kq < 4; ++kq)
                        if (kq == sb) {
                            if (e == 0) sc[kq][0] += part;
                            if (e == 1) sc[kq][1] += part;
                            if (e == 2) sc[kq][2] += part;
                            if (e == 3) sc[kq][3] += part;
                        }
                }
            }
        }
        lds_barrier();   // every wave is done with the raw k rows
    }
    // the state operand into T over the wave's own q rows, the k operand over
    // its own raw k rows
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        st8g<DK>(st.q, 16 * w, 32 * ks, lane, cat(cvt4(Tp[2 * ks]), cvt4(Tp[2 * ks + 1])));
#pragma unroll
    for (int db = 0; db < NDB; ++db) st4g<DK>(st.k, 16 * w, 16 * db, lane, kh[db]);
    lds_barrier();   // (Y) the k operand tile and the state tile are complete

    // the state update, the wave's columns: S <- 2^{a' t} (S 2^{a t} + (k operand)^T V),
    // then the hook (the last chunk publishes the span's summary there). EARLY
    // (one-chunk spans, where the exchange is most of the time): before the
    // scores and outputs, so that the summary travels while they are computed;
    // else after them (fewer registers live across the scores).
    auto state_update = [&]() {
        const h8 vw0 = tr_step<kDV>(st.v, 0, 16 * w, lane), vw1 = tr_step<kDV>(st.v, 1, 16 * w, lane);
#pragma unroll
        for (int it = 0; it < NDB; ++it) {
            Sp[it] = mfma(tr_step<DK>(st.k, 0, 16 * it, lane), vw0, Sp[it]);
            Sp[it] = mfma(tr_step<DK>(st.k, 1, 16 * it, lane), vw1, Sp[it]);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                cs.S[it][e] = Sp[it][e] * (KEEPF ? fbk[it][e] : ex2(be * tot[it][e]));
        }
        after_state(cs);
    };
    if (EARLY) state_update();

    if (!wide) {
        // scores S^T[s][t] for the s-blocks up to the wave's own (lane (n, g):
        // token 16w + n, keys 16 sb + 4 g + e), the diagonal block masked
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            if (sb <= w) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const h8 A = cat(ld4g<DK>(st.k, 16 * sb, 32 * ks, lane),
                                     ld4g<DK>(st.k, 16 * sb, 32 * ks + 16, lane));
                    sc[sb] = mfma(A, qk[ks], sc[sb]);
                }
                if (sb == w) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * g + e > n) sc[sb][e] = 0.f;
                }
            }
        }
    }
    const h8 bs0 = cat(cvt4(sc[0]), cvt4(sc[1]));
    const h8 bs1 = cat(cvt4(sc[2]), cvt4(sc[3]));
    // outputs O^T[j][t]: scores x V (keys up to the wave's block), then the
    // span-local state: state operand x q operand
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        f4 O = mfma(tr_step<kDV>(st.v, 0, 16 * jt, lane), bs0, f4{0.f, 0.f, 0.f, 0.f});
        if (w >= 2) O = mfma(tr_step<kDV>(st.v, 1, 16 * jt, lane), bs1, O);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) O = mfma(ld8g<DK>(st.q, 16 * jt, 32 * ks, lane), qk[ks], O);
        kept.o[jt] = cvt4(O);
    }
    if (!EARLY) state_update();
}

// ---------------------------------------------------------------------------
// Workspace header (gla_ws.h): staged in LDS at the start by wave 0 (a 4-byte
// DMA per lane of lanes 0-3, device scope), checked at the publish.
__device__ __forceinline__ void stage_ws_header(const SpanArgs& a, unsigned int* hdr_lds, int w,
                                                int lane)
{
    if (w == 0 && lane < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(a.hdr, kWsHeaderBytes),
                                                 (__attribute__((address_space(3))) void*)hdr_lds,
                                                 4, 4 * lane, 0, 0, kDevScope);
}
__device__ __forceinline__ bool ws_header_ok(const SpanArgs& a, const unsigned int* hv)
{
    const unsigned int magic = hv[kWsMagicWord];
    return hv[kWsErrWord] == 0 &&
           (magic == kWsClean ||
            (magic == kWsFused && hv[kWsLayoutWord] == a.layout && hv[kWsLayoutCheck] == ~a.layout));
}
// After a successful exchange, workgroup 0 records the layout in a workspace
// that was still clean (every workgroup of the launch has read the header by
// then, or reads either value, which both admit this layout).
__device__ __forceinline__ void mark_ws_header(const SpanArgs& a, const unsigned int* hv, int tid)
{
    if (blockIdx.x == 0 && tid == 0 && hv[kWsMagicWord] == kWsClean) {
        const __amdgpu_buffer_rsrc_t rh = rsrc(a.hdr, kWsHeaderBytes);
        __builtin_amdgcn_raw_buffer_store_b32(a.layout, rh, 4 * kWsLayoutWord, 0, kDevScope);
        __builtin_amdgcn_raw_buffer_store_b32(~a.layout, rh, 4 * kWsLayoutCheck, 0, kDevScope);
        __builtin_amdgcn_raw_buffer_store_b32(kWsFused, rh, 4 * kWsMagicWord, 0, kDevScope);
    }
}

// final_state of sequence seq: DK x 64 fp32 (an empty resource without one)
template <int DK>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t final_rsrc(const SpanArgs& a, int seq)
{
    return rsrc(a.final_state + (a.final_state ? (long long)seq * DK * kDV : 0),
                a.final_state ? DK * kDV * 4 : 0);
}

// Output rows: token t0 + 16w + n, O^T layout (columns 16 jt + 4g .. + 3),
// scaled by d_k^{-1/2}; with a gate, the RMSNorm + SiLU epilogue; poison: NaN.
__device__ __forceinline__ void store_rows(const SpanArgs& a, int b, int h, int t0, int w, int lane,
                                           f4 (&O)[4], bool poison)
{
    const int n = lane & 15, g = lane >> 4;
    const long long per_batch = (long long)a.L * a.H * kDV;
    const int end = (int)(per_batch * 2);
    const int off = pos_bytes<kDV>(a, h, row_pos(a, row_map(a, t0), 16 * w + n), end);
    float f = a.scale;
    u2 z[4];
    if (a.gate) {
        const __amdgpu_buffer_rsrc_t rz = rsrc(a.gate + b * per_batch, end);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            z[jt] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(
                                               rz, off == end ? end : off + 2 * (16 * jt + 4 * g), 0, 0));
        float ss = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += O[jt][e] * O[jt][e];
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        f = a.scale * __builtin_amdgcn_rsqf(a.scale * a.scale * ss * (1.f / kDV) + a.eps);
    }
    if (poison) f = __builtin_nanf("");
    if (off == end) return;
    const __amdgpu_buffer_rsrc_t ro = rsrc(a.out + b * per_batch, end);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
        f4 y = O[jt] * f;
        if (a.gate) {
            const f4 zz = up4(__builtin_bit_cast(h4, z[jt]));
            const f4 ww = *reinterpret_cast<const f4*>(a.norm_w + 16 * jt + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                y[e] = y[e] * ww[e] * zz[e] * __builtin_amdgcn_rcpf(1.f + ex2(-kLog2e * zz[e]));
        }
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u2, cvt4(y)), ro,
                                              off + 2 * (16 * jt + 4 * g), 0, 0);
    }
}

// A launch on an untrusted workspace publishes nothing and waits for nothing:
// it flags the header and writes NaN to every output row of its span and (span
// 0) to the sequence's final state.
template <int DK>
__device__ void fail_untrusted(const SpanArgs& a, int b, int h, int seq, int j, int c_first,
                               int n_c, int w, int lane)
{
    const int tid = 64 * w + lane;
    if (tid == 0) atomicOr(a.hdr + kWsErrWord, kWsErrState);
    for (int c = 0; c < n_c; ++c) {
        f4 O[4];
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) O[jt] = f4{0.f, 0.f, 0.f, 0.f};
        store_rows(a, b, h, (c_first + c) * kC, w, lane, O, true);
    }
    if (j == 0) {
        const __amdgpu_buffer_rsrc_t rf = final_rsrc<DK>(a, seq);
        for (int e = tid; e < DK * kDV; e += kThreads)
            __builtin_amdgcn_raw_buffer_store_b32(0x7FC00000u, rf, 4 * e, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// Value of lane i - N of the same 16-lane row (a lane of the row's first N
// reads 0).
template <int N>
__device__ __forceinline__ float row_shr(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + N, 0xF, 0xF, true));
}
// One step of an inclusive scan over groups of P adjacent lanes (P <= 16, a
// power of two; lane p of its group) of affine maps x -> A x + B, the later
// lane's map applied after the earlier one's.
template <int N>
__device__ __forceinline__ void scan_step(f4& A, f4& B, int p, int P)
{
    if (N >= P) return;   // uniform
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float a2 = row_shr<N>(A[q]), b2 = row_shr<N>(B[q]);
        const bool take = p >= N;
        B[q] = take ? A[q] * b2 + B[q] : B[q];
        A[q] = take ? A[q] * a2 : A[q];
    }
}

// The exchange.
//
// State elements travel in exchange order: element (i, c) of the DK x 64 state
// (i: key dim, c: value column) has index ((i >> 2) << 8) + (c << 2) + (i & 3),
// i.e. row quads, each column's four rows of a quad contiguous. A lane holds
// rows 4q .. 4q + 3 of one column: one 16-byte piece of the summary, one
// 8-byte piece of its incoming state. Owner o folds the elements
// [o 2^lo, (o + 1) 2^lo); its slice covers nr = 2^lr rows (lr = max(2, lo - 6):
// a slice of at most one quad covers that quad's four rows).
//
// Summary words of one sequence, owner-major: owner o's region holds the U
// words of every span [ns][2^lo], then the decays of its rows [ns][nr], padded
// to 16 bytes; the last ranks of the fold read nothing else.
__host__ __device__ inline int slice_rows_log2(int lo) { return lo > 8 ? lo - 6 : 2; }
__host__ __device__ inline int owner_region_words(int ns, int lo)
{
    return (ns << lo) + (((ns << slice_rows_log2(lo)) + 3) & ~3);
}
__device__ __forceinline__ int xelem(int i, int c) { return ((i >> 2) << 8) + (c << 2) + (i & 3); }

// The owner's threads: thread t folds piece t >> (8 - lp) of the slice (4
// elements) over span range t mod P (P = 2^(8 - lp) <= 16 ranges of `per`
// spans; the ranges of a piece sit in adjacent lanes of one 16-lane row), in
// n_pass passes when the slice has more than 256 pieces.
struct FoldMap {
    int lp, P, per, n_pass;
};
__host__ __device__ inline FoldMap fold_map(int ns, int lo)
{
    FoldMap f;
    f.lp = lo - 2 < 8 ? lo - 2 : 8;
    f.P = 1 << (8 - f.lp);
    f.per = (ns + f.P - 1) / f.P;
    f.n_pass = 1 << (lo - 2 - f.lp);
    return f;
}
constexpr int kMaxPer = 8;   // spans per fold range (checked on the host for every plan)

// Publish the span summary U = S (local final state) and D = the span's decay
// as tagged words, straight from the registers: each lane stores its 16-byte
// pieces of U; wave 0 stores the decays of its rows to every owner whose slice
// covers them. Nothing waits for these stores here.
template <int DK>
__device__ __forceinline__ void publish(const SpanArgs& a, const ChunkState<DK>& cs,
                                        long long seq_slot, int j, unsigned int tag, int w, int lane)
{
    constexpr int NDB = DK / 16;
    const int n = lane & 15, g = lane >> 4;
    const int ns = a.n_spans, lo = a.slice_log2, lr = slice_rows_log2(lo);
    const int ow = owner_region_words(ns, lo);
    const __amdgpu_buffer_rsrc_t rs =
        rsrc(a.agg + (seq_slot / ns) * a.agg_words, a.agg_words * 4);
    const int col = 16 * w + n;
#pragma unroll
    for (int it = 0; it < NDB; ++it) {
        const int e = xelem(16 * it + 4 * g, col);
        u4 tw;
#pragma unroll
        for (int k = 0; k < 4; ++k) tw[k] = ll_word(cs.S[it][k], tag);
        __builtin_amdgcn_raw_buffer_store_b128(
            tw, rs, 4 * ((e >> lo) * ow + (j << lo) + (e & ((1 << lo) - 1))), 0, kDevScope);
    }
    if (w == 0) {
        // owners per row quad: 2^(8 - lo) (slices within a quad) or one
        const int nown = lo <= 8 ? 1 << (8 - lo) : 1;
        if (n < nown) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int i = 16 * db + 4 * g;   // rows i .. i + 3
                const int o = lo <= 8 ? ((i >> 2) << (8 - lo)) + n : i >> (lo - 6);
                u4 tw;
#pragma unroll
                for (int k = 0; k < 4; ++k) tw[k] = ll_word((float)cs.Dp[db][k], tag);
                __builtin_amdgcn_raw_buffer_store_b128(
                    tw, rs, 4 * (o * ow + (ns << lo) + (j << lr) + (i & ((1 << lr) - 1))), 0,
                    kDevScope);
            }
        }
    }
}

// Boundary exchange of span j of sequence local_seq: owners fold their slice of
// every span's summary and write each span's incoming state; every workgroup
// then reads its own incoming state into the operand tile sm.tin() ([j][permuted
// i], fp16) and advances its slot's epoch. An owner's thread polls its own
// pieces (device scope) and loads again only those still stale; the fold runs
// on registers. Waits are bounded by a.wait_ticks on the 100 MHz wall clock: a
// wait that passes it gives up (the header's error word records it; an owner
// hands NaN incoming states, with the expected tags, and a NaN final state to
// its slice; a reader that gives up or receives NaN poisons its workgroup's
// outputs). Returns the poison flag.
template <int DK, class L>
__device__ bool exchange(const SpanArgs& a, L& sm, int local_seq, int seq, int j,
                         long long seq_slot, int w, int lane)
{
    constexpr int NE = DK * kDV;             // state elements
    constexpr int kSlot = 2 * NE;            // bytes of one incoming-state slot
    const int tid = 64 * w + lane;
    const int n = lane & 15, g = lane >> 4;
    const int ns = a.n_spans;
    const int lo = a.slice_log2;            // 2^lo elements per owner
    const __amdgpu_buffer_rsrc_t rsl = rsrc(a.sin + seq_slot * kSlot, ns * kSlot);
    if (tid == 0) sm.poison = 0;
    lds_barrier();   // every wave is done with the stages: scratch now
    if (j < (NE >> lo)) {
        const int lr = slice_rows_log2(lo);
        const int ow = owner_region_words(ns, lo);
        const FoldMap f = fold_map(ns, lo);
        const int p = tid & (f.P - 1), pc = tid >> (8 - f.lp);
        const int m_lo = min(p * f.per, ns), m_hi = min(m_lo + f.per, ns);
        const int cnt = m_hi - m_lo;
        const __amdgpu_buffer_rsrc_t rr =
            rsrc(a.agg + local_seq * (long long)a.agg_words + (long long)j * ow, ow * 4);
        const __amdgpu_buffer_rsrc_t rf = final_rsrc<DK>(a, seq);
        float* dl = reinterpret_cast<float*>(sm.region());   // decays [ns][nr] (<= 256)
        const int nd = ns << lr;
        int round = 0;   // poll rounds, counted across the passes (the flags' parity)
        for (int ps = 0; ps < f.n_pass; ++ps) {
            const int el = ((ps << f.lp) + pc) << 2;         // my piece, in the slice
            const int e = (j << lo) + el;                      // ... in the state
            const int i0 = (e >> 8) << 2, col = (e >> 2) & 63; // rows i0 .. i0 + 3, column col
            const int dr = (((e >> 8) - ((j << lo) >> 8)) << 2); // first of my rows, in the slice
            // Every round loads all of my pieces and (wave 0) all of the slice's
            // decay words, with no branches between the loads (a load past the
            // resource reads zero, which no tag accepts; one past my range is
            // not checked), then checks them.
            u4 U[kMaxPer];
            unsigned int tg[kMaxPer];
#pragma unroll
            for (int k = 0; k < kMaxPer; ++k) tg[k] = sm.tags[min(m_lo + k, kMaxSpans - 1)];
            const unsigned long long t_start = now_ticks();
            bool gave_up = false;
            for (;;) {
                asm volatile("" ::: "memory");   // a fresh load every round
#pragma unroll
                for (int k = 0; k < kMaxPer; ++k)
                    U[k] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(
                                                      rr, 4 * (((m_lo + k) << lo) + el), 0, kDevScope));
                unsigned int wd[4];
                if (ps == 0 && w == 0) {   // the slice's decays (the same for all its columns)
#pragma unroll
                    for (int x = 0; x < 4; ++x)
                        wd[x] = __builtin_amdgcn_raw_buffer_load_b32(
                            rr, 4 * ((ns << lo) + lane + 64 * x), 0, kDevScope);
                }
                bool mine = true;
#pragma unroll
                for (int k = 0; k < kMaxPer; ++k) {
                    bool ok = true;
#pragma unroll
                    for (int q = 0; q < 4; ++q) ok = ok && ll_ok(U[k][q], tg[k]);
                    mine = mine && (k >= cnt || ok);
                }
                if (ps == 0 && w == 0) {
#pragma unroll
                    for (int x = 0; x < 4; ++x) {
                        const int dk = lane + 64 * x;
                        const bool ok = dk >= nd || ll_ok(wd[x], sm.tags[min(dk >> lr, kMaxSpans - 1)]);
                        mine = mine && ok;
                        if (dk < nd) dl[dk] = ll_value(wd[x]);
                    }
                }
                // Round r writes the flags of parity r & 1 and reads them after
                // the one barrier; a wave writes that parity again only in round
                // r + 2, after the barrier of round r + 1, which every wave
                // reaches only after reading round r's flags.
                const int pr = round & 1;
                const bool wave_ok = __all(mine);   // (every lane active)
                if (lane == 0) sm.stale_w[pr][w] = wave_ok ? 0 : 1;
                if (tid == 0) sm.expired_r[pr] = (now_ticks() - t_start) > a.wait_ticks ? 1 : 0;
                lds_barrier();
                const bool stale =
                    (sm.stale_w[pr][0] | sm.stale_w[pr][1] | sm.stale_w[pr][2] | sm.stale_w[pr][3]) != 0;
                const bool expired = sm.expired_r[pr] != 0;
                ++round;
                if (!stale) break;
                if (expired) {
                    gave_up = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(kPollSleep);
            }
            // (every load of the poll has returned: said explicitly, so that the
            // stores below are not each made to wait for the ones before them)
            wait_vm0();
            // the slice's initial state (rows i0 .. i0 + 3 of column col)
            f4 s0 = f4{0.f, 0.f, 0.f, 0.f};
            if (a.init) {
                const __amdgpu_buffer_rsrc_t ri = rsrc(a.init + (long long)seq * NE, NE * 4);
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    s0[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        ri, 4 * ((i0 + q) * kDV + col), 0, 0));
            }
            if (gave_up) {
                if (tid == 0) atomicOr(a.hdr + kWsErrWord, kWsErrExchange);
                for (int m = m_lo; m < m_hi; ++m) {
                    // four fp16 NaNs whose lowest bits carry the slot's tag parity
                    const unsigned int hw = 0x7E007E00u | ((sm.tags[m] & 1u) * 0x00010001u);
                    const u2 x = {hw, hw};
                    __builtin_amdgcn_raw_buffer_store_b64(x, rsl, m * kSlot + 2 * e, 0, kDevScope);
                }
                if (p == f.P - 1) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        __builtin_amdgcn_raw_buffer_store_b32(0x7FC00000u, rf,
                                                              4 * ((i0 + q) * kDV + col), 0, 0);
                }
                continue;   // (uniform: every thread of the workgroup gives up together)
            }
            // my range's decays and tag parities, read from LDS once (both
            // passes below then run on registers; the decays are fp16 values,
            // as the spans keep them)
            h4 Dk[kMaxPer];
#pragma unroll
            for (int k = 0; k < kMaxPer; ++k)
                Dk[k] = cvt4(*reinterpret_cast<const f4*>(dl + ((min(m_lo + k, ns - 1)) << lr) + dr));
            // fold my range: product of its decays A and its summary from zero B
            f4 run = f4{0.f, 0.f, 0.f, 0.f};
            if (f.P > 1) {
                f4 A = f4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int k = 0; k < kMaxPer; ++k) {
                    const bool in = k < cnt;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float d = (float)Dk[k][q];
                        A[q] = in ? A[q] * d : A[q];
                        run[q] = in ? d * run[q] + ll_value(U[k][q]) : run[q];
                    }
                }
                // the ranges before mine, from the initial state: an exclusive
                // scan of the (A, B) pairs over the piece's adjacent lanes
                // (compose: a later range (A, B) after an earlier (A', B') is
                // (A A', A B' + B))
                scan_step<1>(A, run, p, f.P);
                scan_step<2>(A, run, p, f.P);
                scan_step<4>(A, run, p, f.P);
                scan_step<8>(A, run, p, f.P);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    // (the shifts run in every lane, before the select: a lane
                    // reading one masked off would read zero)
                    const float sa = row_shr<1>(A[q]), sb = row_shr<1>(run[q]);
                    const float xa = p > 0 ? sa : 1.f;
                    const float xb = p > 0 ? sb : 0.f;
                    run[q] = xa * s0[q] + xb;
                }
            } else {
                run = s0;
            }
            // my range again, storing each span's incoming state; the last range
            // ends with the final state
#pragma unroll
            for (int k = 0; k < kMaxPer; ++k) {
                if (k < cnt) {
                    const unsigned int t1 = tg[k] & 1u;
                    u2 x;
                    x[0] = (unsigned int)sin_word(run[0], t1) | ((unsigned int)sin_word(run[1], t1) << 16);
                    x[1] = (unsigned int)sin_word(run[2], t1) | ((unsigned int)sin_word(run[3], t1) << 16);
                    __builtin_amdgcn_raw_buffer_store_b64(x, rsl, (m_lo + k) * kSlot + 2 * e, 0,
                                                          kDevScope);
#pragma unroll
                    for (int q = 0; q < 4; ++q) run[q] = (float)Dk[k][q] * run[q] + ll_value(U[k][q]);
                }
            }
            if (p == f.P - 1) {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(run[q]), rf,
                                                          4 * ((i0 + q) * kDV + col), 0, 0);
            }
        }
    }

    // my incoming state: each wave polls its pieces (rows 16 it + 4 g .. + 3,
    // column 16w + n) until every word carries the slot's tag, then writes them
    // to the operand tile in the permuted order; span 0 reads its zeros like
    // the others so that its epoch, too, advances only once every owner has
    // read it
    {
        constexpr int NDB = DK / 16, NKS = DK / 32;
        const unsigned int tag = sm.tags[j];
        const int col = 16 * w + n;
        const unsigned long long t_start = now_ticks();
        bool bad = false;
        h4 x[NDB];
        for (;;) {
            asm volatile("" ::: "memory");   // a fresh load every round
            u2 u[NDB];
#pragma unroll
            for (int it = 0; it < NDB; ++it)
                u[it] = __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(
                                                   rsl, j * kSlot + 2 * xelem(16 * it + 4 * g, col), 0,
                                                   kDevScope));
            bool ok = true;
#pragma unroll
            for (int it = 0; it < NDB; ++it)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const unsigned short hw = (unsigned short)(u[it][q >> 1] >> (16 * (q & 1)));
                    ok &= sin_ok(hw, tag);
                    x[it][q] = sin_value(hw);
                }
            if (__all(ok)) break;
            if (now_ticks() - t_start > a.wait_ticks) {   // wave-uniform
                if (lane == 0) atomicOr(a.hdr + kWsErrWord, kWsErrExchange);
                bad = true;
                break;
            }
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
#pragma unroll
        for (int it = 0; it < NDB; ++it)
#pragma unroll
            for (int q = 0; q < 4; ++q) bad |= __builtin_isnan((float)x[it][q]);
        if (__any(bad) && lane == 0) sm.poison = 1;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            st8g<DK>(sm.tin(), 16 * w, 32 * ks, lane, cat(x[2 * ks], x[2 * ks + 1]));
        // Every owner has read this slot's epoch (it wrote S_in after reading
        // the epochs), and so has every wave here: advance it.
        lds_barrier();
        if (tid == 0)
            __hip_atomic_store(a.epoch + seq_slot + j, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return sm.poison != 0;
}


// ---------------------------------------------------------------------------
// The kernel. VAR 0: plain; 1: with an initial state and/or the output gate
// (the plain kernel's copy of the arguments has constant nulls for them).
// Spans short enough that per-chunk constants of a lane (the prefix operand,
// the row factor) stay in registers across the chunk instead of being rebuilt.
template <int DK, int SPAN>
constexpr bool kHoist = DK == 32 || SPAN <= 4;

// Two workgroups per CU (256 registers per lane): the exchange's fold holds a
// range of summaries in registers next to the kept outputs.
template <int DK, int SPAN, int VAR>
__global__ void __launch_bounds__(kThreads, 2)
gla_span_kernel(SpanArgs a_arg)
{
    constexpr int NDB = DK / 16, NKS = DK / 32;
    constexpr int NS = SPAN > 1 ? 2 : 1;
    {
        // one word of each 64-byte line of the arguments, in one batch: every
        // later argument load hits the scalar cache
        const unsigned int* aw = reinterpret_cast<const unsigned int*>(&a_arg);
        asm volatile("" ::"s"(aw[0]), "s"(aw[16]), "s"(aw[32]));
    }
    SpanArgs a = a_arg;
    if (VAR == 0) {
        a.init = nullptr;
        a.gate = nullptr;
    }
    __shared__ Lds<DK, NS> sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane0 = tid & 63;
    const int local_seq = blockIdx.x / a.n_spans;
    const int j = blockIdx.x - local_seq * a.n_spans;
    const int seq = a.seq0 + local_seq;
    const int b = seq / a.H, h = seq - b * a.H;
    const int c_first = j * SPAN;
    const int n_c = min(SPAN, a.n_chunks - c_first);
    const long long seq_slot = (long long)local_seq * a.n_spans;

    // epochs of the sequence's span slots (thread t < n_spans: slot t), the
    // workspace header, the first chunk: all in flight
    const unsigned int ep = __builtin_amdgcn_raw_buffer_load_b32(
        rsrc(a.epoch + seq_slot, 4 * a.n_spans), 4 * tid, 0, kDevScope);
    stage_ws_header(a, sm.hdr, w, lane0);
    dma_stage(a, sm.stage[0], b, h, c_first * kC, w, lane0);
    ChunkState<DK> cs;
#pragma unroll
    for (int it = 0; it < NDB; ++it) {
        cs.S[it] = f4{0.f, 0.f, 0.f, 0.f};
        cs.Dp[it] = h4{(_Float16)1.f, (_Float16)1.f, (_Float16)1.f, (_Float16)1.f};
    }

    // ---- 1. local pass: SPAN chunks, always (past the sequence end the rows
    // read zeros: the state and the decay stay, the outputs are not stored)
    Kept<DK> kept[SPAN];
#pragma unroll 1
    for (int c = 0; c < SPAN; ++c) {
        // the lane index passes through an empty asm each chunk, so that the
        // lane-dependent LDS and global addresses are recomputed where they are
        // used instead of being hoisted out of the loop and held in registers
        int lane = lane0;
        asm volatile("" : "+v"(lane));
        wait_vm0();
        lds_barrier();   // (X) chunk c is staged; chunk c - 1's tiles are free
        if (c == 0 && tid < kMaxSpans)   // seen by every wave after the chunk's next barrier
            sm.tags[tid] = (ep + 1u) & 0xFFu;
        if (c + 1 < SPAN)   // wave-uniform
            dma_stage(a, sm.stage[(c + 1) & (NS - 1)], b, h, (c_first + c + 1) * kC, w, lane);
        auto& st = sm.stage[c & (NS - 1)];
        f4 bsum[NDB], tot[NDB];
        // the 0/1 operand of the gate prefix depends on the lane and the wave
        // only: built once before the loop (from the lane index that is not
        // recomputed per chunk) where the registers allow, else per chunk
        chunk_gates<DK>(st.g, w, lane, kHoist<DK, SPAN> ? lane0 : lane, bsum, tot);
        bool wide = false;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e) wide |= tot[db][e] < -kGuard / kLog2e;
        Kept<DK> kc_out;
        // every wave sees the same totals: the decision is the same in every wave
        // the last chunk publishes the span's summary as soon as its state
        // update is done (a workspace the header does not admit gets no
        // publish; the test hook silences span 0)
        // (one-chunk spans only; longer ones publish after the loop, which keeps
        // the publish's registers out of the chunk loop)
        auto publish_last = [&](const ChunkState<DK>& s_) {
            if (SPAN == 1 && ws_header_ok(a, sm.hdr) && !(a.fault && j == 0))   // uniform
                publish<DK>(a, s_, seq_slot, j, sm.tags[j], w, lane);
        };
        chunk_step<DK, kHoist<DK, SPAN>, SPAN == 1>(st, w, lane, bsum, tot, __any(wide), cs, kc_out,
                                                    publish_last);
#pragma unroll
        for (int i = 0; i < SPAN; ++i)
            if (i == c) kept[i] = kc_out;   // c is wave-uniform: a scalar branch
    }
    const int lane = lane0;
    const int n = lane & 15, g = lane >> 4;

    // ---- 2. publish and exchange (the header, staged at the start, has landed:
    // wave 0 waited for it before the first chunk's barrier; every wave reads
    // the same words, so the decision is the workgroup's)
    if (!ws_header_ok(a, sm.hdr)) {   // (published nothing)
        fail_untrusted<DK>(a, b, h, seq, j, c_first, n_c, w, lane);
        return;
    }
    if (SPAN > 1 && !(a.fault && j == 0)) publish<DK>(a, cs, seq_slot, j, sm.tags[j], w, lane);
    const bool has_in = j > 0 || a.init != nullptr;
    const bool poison = exchange<DK>(a, sm, local_seq, seq, j, seq_slot, w, lane);
    if (!poison) mark_ws_header(a, sm.hdr, tid);

    // ---- 3. outputs: kept + (q 2^b D_c) S_in
    const _Float16* tin = sm.tin();
#pragma unroll
    for (int c = 0; c < SPAN; ++c) {
        if (c < n_c) {
            f4 O[4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) O[jt] = up4(kept[c].o[jt]);
            if (has_in) {
#pragma unroll
                for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        O[jt] = mfma(ld8g<DK>(tin, 16 * jt, 32 * ks, lane), kept[c].qs[ks], O[jt]);
            }
            store_rows(a, b, h, (c_first + c) * kC, w, lane, O, poison);
        }
    }
}

}  // namespace span

// ---------------------------------------------------------------------------
// host side

namespace {

using span::gla_span_kernel;

template <int DK, int VAR>
const void* span_kernel_v(int sp)
{
    switch (sp) {
    case 1: return (const void*)gla_span_kernel<DK, 1, VAR>;
    case 2: return (const void*)gla_span_kernel<DK, 2, VAR>;
    case 3: return (const void*)gla_span_kernel<DK, 3, VAR>;
    case 4: return (const void*)gla_span_kernel<DK, 4, VAR>;
    case 5: return (const void*)gla_span_kernel<DK, 5, VAR>;
    case 6: return (const void*)gla_span_kernel<DK, 6, VAR>;
    default: return (const void*)gla_span_kernel<DK, 7, VAR>;
    }
}
const void* span_kernel(int dk, int sp, int var)
{
    if (dk == 32) return var ? span_kernel_v<32, 1>(sp) : span_kernel_v<32, 0>(sp);
    return var ? span_kernel_v<64, 1>(sp) : span_kernel_v<64, 0>(sp);
}

int span_resident_per_cu(int dk, int sp, int var)
{
    static int cache[2][span::kMaxSpan + 1][2] = {};
    int& c = cache[dk == 32 ? 0 : 1][sp][var ? 1 : 0];
    if (c == 0) {
        int n = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, span_kernel(dk, sp, var), span::kThreads, 0);
        if (e != hipSuccess) {
            log_hip("occupancy query of a span kernel", e);
            (void)hipGetLastError();   // do not leave it for a later call to report
            n = 1;                     // one per CU: every kernel here fits that
        }
        if (n < 1) n = 1;
        c = n;
    }
    return c;
}

int span_device_cus()
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

size_t a256(size_t x) { return (x + 255) / 256 * 256; }

// owners: the largest power of two <= n_spans, at most one per state row
int span_slice_log2(int dk, int n_spans)
{
    const int ne = dk * 64;
    int owners = 1;
    while (owners * 2 <= n_spans && owners * 2 <= ne / 64) owners *= 2;
    int lo = 0;
    while ((1 << lo) < ne / owners) ++lo;
    return lo;
}
int span_agg_words(int dk, int n_spans, int lo)
{
    const int owners = (dk * 64) >> lo;
    return (owners * span::owner_region_words(n_spans, lo) + 63) / 64 * 64;
}
// the exchange's fold: at most kMaxPer spans per range of one thread, at most
// 256 decay words per slice
bool span_exchange_ok(int dk, int sp, int n_spans, int lo)
{
    (void)dk;
    (void)sp;
    return lo >= 6 && span::fold_map(n_spans, lo).per <= span::kMaxPer &&
           (n_spans << span::slice_rows_log2(lo)) <= 256;   // the slice's decays, in LDS
}

}  // namespace

bool span_supported(const Shape& s)
{
    return (s.d_k == 64 || s.d_k == 32) && s.d_v == 64 && s.chunk == 64 &&
           (long long)s.L * s.H * 64 * 2 + 256 <= 0x7FFFFFFFLL &&
           s.n_chunks <= span::kMaxSpan * span::kMaxSpans;
}

FusedPlan span_plan(const Shape& s, int span_override, long long cap_override, int var)
{
    FusedPlan p{};
    p.family = 2;
    p.dk = s.d_k;   // the state rows set the exchange's slot layout (and its layout word)
    p.keep = true;
    p.rk = false;
    p.var = var;
    const int n_seq = s.B * s.H;
    const int nc = s.n_chunks;
    auto fill = [&](int sp) {
        p.span = sp;
        p.n_spans = (nc + sp - 1) / sp;
        long long cap = resident_cap(span_resident_per_cu(s.d_k, sp, var), span_device_cus());
        if (cap_override > 0 && cap_override < cap) cap = cap_override;
        long long per = cap / p.n_spans;
        if (per < 1) per = 1;
        p.seq_batch = (int)(per < n_seq ? per : n_seq);
        p.grid = p.seq_batch * p.n_spans;
        p.slice_log2 = span_slice_log2(s.d_k, p.n_spans);
        return (long long)p.n_spans <= cap && p.n_spans <= span::kMaxSpans &&
               span_exchange_ok(s.d_k, sp, p.n_spans, p.slice_log2);
    };
    if (span_override >= 1 && span_override <= span::kMaxSpan && fill(span_override)) return p;
    // the shortest span whose whole call is resident at once, else the shortest
    // whose one sequence is (several launches)
    for (int sp = 1; sp <= span::kMaxSpan; ++sp)
        if (fill(sp) && p.seq_batch == n_seq) return p;
    for (int sp = 1; sp <= span::kMaxSpan; ++sp)
        if (fill(sp)) return p;
    p.family = 0;   // no span plan: the caller takes another kernel
    return p;
}

size_t span_workspace_bytes(const Shape& s, const FusedPlan& p)
{
    const size_t slots = (size_t)p.seq_batch * p.n_spans;
    const size_t ne = (size_t)s.d_k * 64;
    return kWsHeaderBytes + a256(slots * 4) +
           a256((size_t)p.seq_batch * span_agg_words(s.d_k, p.n_spans, p.slice_log2) * 4) +
           a256(slots * 2 * ne);
}

hipError_t launch_span(const void* q, const void* k, const void* v, const void* lg, const Shape& s,
                       const Extras& x, const FusedPlan& p, void* out, float* final_state,
                       void* ws, hipStream_t st, unsigned int layout, int fault,
                       unsigned long long wait_ticks)
{
    if (p.family != 2 || p.span < 1 || p.span > span::kMaxSpan) return hipErrorInvalidValue;
    if (p.var == 0 && (x.init || x.gate)) return hipErrorInvalidValue;
    if (x.z) return hipErrorInvalidValue;   // the low-rank gate runs on the other kernels
    if (!span_exchange_ok(s.d_k, p.span, p.n_spans, p.slice_log2)) return hipErrorInvalidValue;
    span::SpanArgs a;
    a.q = (const __half*)q;
    a.k = (const __half*)k;
    a.v = (const __half*)v;
    a.lg = (const __half*)lg;
    a.out = (__half*)out;
    a.final_state = final_state;
    unsigned char* base = (unsigned char*)ws;
    const size_t slots = (size_t)p.seq_batch * p.n_spans;
    a.hdr = (unsigned int*)base;
    a.epoch = (unsigned int*)(base + kWsHeaderBytes);
    a.agg_words = span_agg_words(s.d_k, p.n_spans, p.slice_log2);
    a.agg = (unsigned int*)(base + kWsHeaderBytes + a256(slots * 4));
    a.sin = (unsigned char*)a.agg + a256((size_t)p.seq_batch * a.agg_words * 4);
    a.L = s.L;
    a.H = s.H;
    a.grid_h = s.grid_h;
    a.grid_w = s.grid_w;
    a.dir = s.dir;
    a.n_chunks = s.n_chunks;
    a.n_spans = p.n_spans;
    a.slice_log2 = p.slice_log2;
    a.scale = s.scale;
    a.inv_gh = 1.0f / (float)s.grid_h;
    a.init = x.init;
    a.gate = (const __half*)x.gate;
    a.norm_w = x.norm_w;
    a.eps = x.eps;
    a.layout = layout;
    a.fault = fault;
    a.wait_ticks = wait_ticks;
    const void* fn = span_kernel(s.d_k, p.span, p.var);
    const int n_seq = s.B * s.H;
    for (int s0 = 0; s0 < n_seq; s0 += p.seq_batch) {
        a.seq0 = s0;
        const int nseq = (n_seq - s0 < p.seq_batch) ? (n_seq - s0) : p.seq_batch;
        void* args[] = {&a};
        const hipError_t e = hipLaunchKernel(fn, dim3(nseq * p.n_spans), dim3(span::kThreads), args,
                                             0, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gtrgla
