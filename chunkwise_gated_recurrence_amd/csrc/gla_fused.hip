// gla_fused.hip -- the fused fp16 path for d_k = d_v = 64, chunk C = 64, on
// gfx950 (CDNA4) MFMA.
//
// It evaluates the chunkwise form of key-only GLA (GTR summary page
// "GTR:门控Token循环实现高效稠密预测", section 前置知识 › Chunkwise(分块)并行; the
// operator of its section 方法步骤详情, and section 3.3 of the 0539edu.com
// page): per-chunk summaries U_c and decays d_c, the boundary scan
// S_[c+1] = Diag(d_c) S_[c] + U_c, and per-chunk outputs.
//
// Work decomposition. Every (batch, head) sequence is cut into n_spans spans
// of `span` consecutive 64-token chunks, one workgroup (4 waves) per span, and
// every workgroup of a launch is resident at once (the host sizes spans and
// sequence batches so that it is).
//   1. Local pass over the span's chunks, streamed once from HBM with the scan
//      direction folded into the row addresses. The state starts at zero at
//      the span start. With KEEP the pass also computes every chunk's outputs
//      and keeps them (and the q 2^b operands) in registers; without KEEP it
//      only accumulates the span summary.
//   2. Boundary scan across spans, in two device-wide exchanges: every
//      workgroup publishes its span summary (D = product of gates, U = local
//      final state); workgroup j then scans a 1/n_spans slice of the 64x64
//      state elements through all spans of its sequence and publishes the
//      incoming state of every span for that slice; each workgroup then reads
//      its own incoming state S_in.
//   3. With KEEP: add (q_t 2^{b_t}) Diag(2^{P_c}) S_in to the kept outputs and
//      store them. Without KEEP: stream the span again (mostly from cache)
//      starting from S_in and store the outputs as they are produced.
//
// Exchanged values travel as 8-byte words {float value, 32-bit tag} written
// and read with device-scope (sc1) accesses. A reader polls the words
// themselves until every tag equals this launch's tag, so a hand-over costs
// one memory round trip: no flags, no fences, no atomics. The tag is a
// per-sequence epoch kept in the workspace, advanced once per launch, so a
// workspace is cleared only once.
//
// Per chunk (wave w owns rows 16w..16w+15 of the chunk and state rows
// 16w..16w+15; lane l holds row r = l & 15 and dims 8(l >> 4) + 32h + e):
//   * loads land directly in the MFMA operand layout (16 B per lane);
//   * log2-gate prefix: a 16-lane DPP row scan; 64 threads then turn the four
//     wave totals into per-dim offsets and constants shared through LDS;
//   * E = 2^{b - r}: q E (= q 2^{b-r}) and q E 2^r (= q 2^b) stay in registers
//     as MFMA operands, k / E goes to LDS for the other waves, and
//     (k / E) 2^{b_last - r} and v are transposed by an MFMA against a 0/1
//     selector (exact) and stored with 8-byte writes;
//   * MFMA 16x16x32 fp16 -> fp32: scores, scores x V, (q 2^b) x S and
//     (k 2^{b_last-b})^T x V for the state update.
// Scores use the factorisation (Q 2^{B-r})(K 2^{r-B})^T, r the middle of the
// chunk's log2-gate range, valid when that range is <= kGuard (every factor
// then lies in [2^-8, 2^8]). A chunk with a wider range (very strong decay)
// computes its scores exactly in fp32 instead.
#include "gla_common.h"
#include "gla_launch.h"

namespace gtrgla {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

constexpr int kC = 64;            // chunk length
constexpr int kD = 64;            // d_k = d_v
constexpr int kThreads = 256;     // 4 waves
constexpr int kMaxKeep = 2;       // longest span kept on chip
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGuard = 16.0f;   // max log2 range of a chunk for factorised scores
constexpr int kTile = kC * 72;    // halves per LDS tile (rows padded to 72)
constexpr int kAggWords = kD * kD + kD;   // U (lane order) then D
constexpr unsigned int kMaxPolls = 1u << 22;
constexpr int kMaxSpans = 64;        // spans per sequence
constexpr int kScanU = 40 * 1024;    // exchange scratch: span words of a slice
constexpr int kScanD = 512;          // exchange scratch: decays of a slice (floats)
constexpr int kDevScope = 16;        // cache policy: device-scope (sc1) access

// ---------------------------------------------------------------------------
// small device helpers

// 64 x 64 fp16 tiles in LDS with rows padded to 72 halves (144 B): the 16 rows
// an MFMA operand read touches fall on distinct banks, and every access is a
// per-lane base plus a compile-time offset.
constexpr int kRow = 72;
__device__ __forceinline__ h8 ld8(const _Float16* t, int row, int col)
{
    return *reinterpret_cast<const h8*>(t + row * kRow + col);
}
__device__ __forceinline__ void st8(_Float16* t, int row, int col, h8 x)
{
    *reinterpret_cast<h8*>(t + row * kRow + col) = x;
}
__device__ __forceinline__ void st4(_Float16* t, int row, int col, h4 x)
{
    *reinterpret_cast<h4*>(t + row * kRow + col) = x;
}

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Barrier that orders LDS only: outstanding global loads stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int N>
__device__ __forceinline__ float row_shr(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 0x110 + N, 0xF, 0xF, true));
}

// Hardware 2^x and 1/x (about 1 ulp).
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Tagged exchange words.
__device__ __forceinline__ void ll_store(u64* p, float v, unsigned int tag)
{
    __hip_atomic_store(p, ((u64)tag << 32) | (u64)__float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool ll_load(const u64* p, unsigned int tag, float& v)
{
    const u64 x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    v = __uint_as_float((unsigned int)x);
    return (unsigned int)(x >> 32) == tag;
}

__device__ __forceinline__ void unpack8(u4 u, float* f)
{
    const h8 h = __builtin_bit_cast(h8, u);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (float)h[e];
}
__device__ __forceinline__ h8 pack8(const float* f)
{
    h8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)f[e];
    return r;
}
__device__ __forceinline__ h4 pack4(f4 x, float s)
{
    h4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = (_Float16)(x[e] * s);
    return r;
}
__device__ __forceinline__ void ld_f8(const float* p, float* f)
{
    const f4 a = *reinterpret_cast<const f4*>(p);
    const f4 b = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = a[e];
        f[4 + e] = b[e];
    }
}

// 0/1 selector (B operand of a 32x16 block): B[k][n] = (k == n + 16 half).
__device__ __forceinline__ h8 selector(int lane, int half)
{
    h8 s;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        s[e] = (_Float16)((8 * (lane >> 4) + e == (lane & 15) + 16 * half) ? 1.0f : 0.0f);
    return s;
}

// ---------------------------------------------------------------------------
struct FusedArgs {
    const __half* q;
    const __half* k;
    const __half* v;
    const __half* lg;
    __half* out;
    float* final_state;
    unsigned int* epoch;        // [seq in launch] launches completed
    unsigned int* err;          // set when a wait gives up
    u64* agg;                   // [seq in launch][n_spans][kAggWords]  tagged
    u64* sin;                   // [seq in launch][n_spans][kD * kD]   tagged
    int L, H, grid_h, grid_w, dir;
    int n_chunks;               // per sequence
    int span;                   // chunks per workgroup
    int n_spans;                // workgroups per sequence
    int seq0;                   // first sequence of this launch
    int slice;                  // state elements per workgroup in the scan
    float scale;
};

struct Smem {
    // Kh and Sc are adjacent: the exact-score path uses them as one fp32 table.
    // Kh .. ST0 (five tiles) also serve as the exchange scratch.
    _Float16 Kh[kTile];       // k 2^{r-b}, rows s
    _Float16 Sc[kTile];       // per-wave rows: scores [t][s], then output staging [t][j]
    _Float16 KtT[kTile];      // (k 2^{b_last-b})^T  [i][s]   (exact path: raw k)
    _Float16 VT[kTile];       // v^T                 [j][s]
    _Float16 ST0[kTile];      // fp16 state, transposed [j][i]
    float tot[4][kD];         // per-wave sums of log2 gates
    float bfirst[kD];         // log2 gate of the chunk's first row
    float pre[4][kD];         // prefix offset of each wave's rows
    float ref[kD];            // reference point r
    _Float16 cq16[kD];        // 2^r
    _Float16 ck16[kD];        // 2^{b_last - r}
    float dcv[kD];            // 2^{b_last} = d_c
    float blast[kD];          // b_last (log2 of d_c)
    float P[kMaxKeep + 1][kD];  // log2 decay from the span start to each chunk start
    float Pend[kD];           // log2 decay of the span so far
    unsigned int tag;
    int fail;
    int stale;
    _Float16 ST1[kTile];      // second state buffer, last: one-chunk spans never use it
};

__device__ __forceinline__ _Float16* st_tile(Smem& sm, int i) { return i ? sm.ST1 : sm.ST0; }

struct ChunkRegs {
    u4 q[2], k[2], v[2], g[2];
};

// Row offset (halves) of scan step t of sequence (b, h); -1 past the end.
__device__ __forceinline__ long long row_offset(const FusedArgs& a, int b, int h, int t)
{
    if (t >= a.L) return -1;
    const int p = scan_to_spatial(t, a.L, a.grid_h, a.grid_w, a.dir);
    return (((long long)b * a.L + p) * a.H + h) * kD;
}

__device__ __forceinline__ u4 load16(const __half* base, long long off)
{
    if (off < 0) return u4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load(reinterpret_cast<const u4*>(base + off));
}

// Lane l of wave w loads row 16w + (l & 15), dims 8(l >> 4) + 32h .. +7.
template <bool WITH_Q>
__device__ __forceinline__ void load_chunk(const FusedArgs& a, int b, int h, int t0, int w,
                                           int lane, ChunkRegs& R)
{
    const long long off = row_offset(a, b, h, t0 + 16 * w + (lane & 15));
    const int col = 8 * (lane >> 4);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const long long o = off < 0 ? -1 : off + col + 32 * hh;
        if (WITH_Q) R.q[hh] = load16(a.q, o);
        R.k[hh] = load16(a.k, o);
        R.v[hh] = load16(a.v, o);
        R.g[hh] = load16(a.lg, o);
    }
}

// Exact fp32 scores of the wave's rows t = 16w + r for a chunk whose gate
// range is too wide for the factorised form. The fp32 prefix of every row goes
// to the Kh+Sc table and raw k to KtT (the state update has consumed it); each
// lane sums its own 16 dims and four lanes (one per dim group) combine.
__device__ void exact_scores(Smem& sm, const ChunkRegs& R, const float (&x)[2][8], int w,
                             int lane, f4 (&sc)[4])
{
    const int r = lane & 15, g = lane >> 4;
    const int t = 16 * w + r;
    float* Bt = reinterpret_cast<float*>(sm.Kh);       // [64][64] fp32, overlays Kh and Sc
    _Float16* Kr = sm.KtT;                             // [64][64] raw k, row-major
    lds_barrier();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int e = 0; e < 8; ++e) Bt[t * kD + 32 * hh + 8 * g + e] = x[hh][e];
        *reinterpret_cast<u4*>(Kr + t * kD + 32 * hh + 8 * g) = R.k[hh];
    }
    lds_barrier();
    float qf[2][8];
    unpack8(R.q[0], qf[0]);
    unpack8(R.q[1], qf[1]);
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) sc[sb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int s = 0; s <= 16 * w + 15; ++s) {
        float part = 0.f;
        if (s <= t) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                float bs[8], kf[8];
                ld_f8(Bt + s * kD + 32 * hh + 8 * g, bs);
                unpack8(*reinterpret_cast<const u4*>(Kr + s * kD + 32 * hh + 8 * g), kf);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    part += qf[hh][e] * kf[e] * ex2(fminf(x[hh][e] - bs[e], 0.f));
            }
        }
        // sum over the four dim groups (lanes r, r+16, r+32, r+48)
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        // lane (r, g) keeps s = 16 sb + 4 g + e
        const int sb = s >> 4, rem = s & 15;
        if ((rem >> 2) == g) {
            const int e = rem & 3;
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                if (q4 == sb) {
                    if (e == 0) sc[q4][0] = part;
                    if (e == 1) sc[q4][1] = part;
                    if (e == 2) sc[q4][2] = part;
                    if (e == 3) sc[q4][3] = part;
                }
        }
    }
    lds_barrier();
}

// What the output half of a chunk needs from its front half.
struct ChunkTmp {
    h8 qh[2];        // q 2^{b-r} (factorised scores)
    float x[2][8];   // log2 prefix b (exact scores)
    bool exact;
};

// Front half of one chunk: log2-gate prefix, per-dim constants, operand tiles,
// and the state update S <- Diag(d_c) S + (k 2^{b_last-b})^T v. S (C layout:
// rows 16w+4g+e, cols 16jt+r) enters as the state at the chunk start and
// leaves as the state after it; written transposed to ST[st ^ 1] when
// write_next. FULL also prepares the output half (Qt = q 2^b, Kh, qh).
template <bool FULL>
__device__ __forceinline__ void chunk_front(Smem& sm, const ChunkRegs& R, int w, int lane, int c,
                                            f4 (&S)[4], int st, bool write_next, h8 (&Qt)[2],
                                            ChunkTmp& T)
{
    const int r = lane & 15, g = lane >> 4;
    const int tid = 64 * w + lane;

    // -- log2 gates, inclusive prefix over the wave's 16 rows
    float x[2][8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        unpack8(R.g[hh], x[hh]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float y = x[hh][e] * kLog2e;
            y += row_shr<1>(y);
            y += row_shr<2>(y);
            y += row_shr<4>(y);
            y += row_shr<8>(y);
            x[hh][e] = y;
        }
    }
    if (r == 15) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.tot[w][32 * hh + 8 * g + e] = x[hh][e];
    }
    if (w == 0 && r == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.bfirst[32 * hh + 8 * g + e] = x[hh][e];
    }
    lds_barrier();  // (A)

    // -- per-dim offsets and constants, one thread per key dim
    if (tid < kD) {
        const int d = tid;
        const float t0 = sm.tot[0][d], t1 = sm.tot[1][d], t2 = sm.tot[2][d], t3 = sm.tot[3][d];
        sm.pre[0][d] = 0.f;
        sm.pre[1][d] = t0;
        sm.pre[2][d] = t0 + t1;
        sm.pre[3][d] = t0 + t1 + t2;
        const float bl = t0 + t1 + t2 + t3;
        const float bf = sm.bfirst[d];
        const float rf = 0.5f * (bf + bl);
        sm.ref[d] = rf;
        sm.cq16[d] = (_Float16)ex2(rf);
        sm.ck16[d] = (_Float16)ex2(bl - rf);
        sm.dcv[d] = ex2(bl);
        sm.blast[d] = bl;
        sm.Pend[d] += bl;
        if (c < kMaxKeep) sm.P[c + 1][d] = sm.P[c][d] + bl;
        const bool wide = __any((bf - bl) > kGuard);
        if (d == 0) sm.fail = wide ? 1 : 0;
    }
    lds_barrier();  // (A2)

    const bool exact = FULL && sm.fail;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int d0 = 32 * hh + 8 * g;
        float pre[8];
        ld_f8(&sm.pre[w][d0], pre);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[hh][e] += pre[e];
        h8 kt8;
        if (FULL && !exact) {
            // E = 2^{b-r} and 1/E in fp32, the products in packed fp16
            float rf[8], ef[8], ei[8];
            ld_f8(&sm.ref[d0], rf);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dlt = x[hh][e] - rf[e];
                ef[e] = ex2(dlt);
                ei[e] = ex2(-dlt);
            }
            const h8 cq = *reinterpret_cast<const h8*>(&sm.cq16[d0]);
            const h8 ck = *reinterpret_cast<const h8*>(&sm.ck16[d0]);
            const h8 q8 = __builtin_bit_cast(h8, R.q[hh]);
            const h8 k8 = __builtin_bit_cast(h8, R.k[hh]);
            const h8 qh = q8 * pack8(ef);
            const h8 kh = k8 * pack8(ei);
            T.qh[hh] = qh;
            Qt[hh] = qh * cq;
            kt8 = kh * ck;
            st8(sm.Kh, 16 * w + r, d0, kh);
        } else {
            float bl[8], kf[8], kt[8];
            ld_f8(&sm.blast[d0], bl);
            unpack8(R.k[hh], kf);
#pragma unroll
            for (int e = 0; e < 8; ++e) kt[e] = kf[e] * ex2(bl[e] - x[hh][e]);
            kt8 = pack8(kt);
            if (FULL) {
                float qf[8], q2[8];
                unpack8(R.q[hh], qf);
#pragma unroll
                for (int e = 0; e < 8; ++e) q2[e] = qf[e] * ex2(x[hh][e]);
                Qt[hh] = pack8(q2);
            }
        }
        // transposes through the MFMA: D[m][n] = X[16w + m][32hh + 16half + n]
        const h8 v8 = __builtin_bit_cast(h8, R.v[hh]);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const f4 zero = {0.f, 0.f, 0.f, 0.f};
            const h8 sel = selector(lane, half);
            const f4 dk = mfma(kt8, sel, zero);
            const f4 dv = mfma(v8, sel, zero);
            const int row = 32 * hh + 16 * half + r;
            st4(sm.KtT, row, 16 * w + 4 * g, pack4(dk, 1.f));
            st4(sm.VT, row, 16 * w + 4 * g, pack4(dv, 1.f));
        }
    }
    lds_barrier();  // (B)

    // -- state: S[i][j] <- d_c[i] S[i][j] + sum_s KtT[i][s] VT[j][s]
    const f4 dc = *reinterpret_cast<const f4*>(&sm.dcv[16 * w + 4 * g]);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) S[jt][e] *= dc[e];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            S[jt] = mfma(ld8(sm.KtT, 16 * w + r, 32 * ks + 8 * g),
                         ld8(sm.VT, 16 * jt + r, 32 * ks + 8 * g), S[jt]);
    }
    if (write_next) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            st4(st_tile(sm, st ^ 1), 16 * jt + r, 16 * w + 4 * g, pack4(S[jt], 1.f));
    }
    if (FULL) {
        T.exact = exact;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) T.x[hh][e] = x[hh][e];
    }
}

// Output half of one chunk: O^T[j][t] += sum_s VT[j][s] Sc[t][s], plus
// sum_i ST[st][j][i] Qt[t][i] when has_state.
__device__ __forceinline__ void chunk_back(Smem& sm, const ChunkRegs& R, int w, int lane, int st,
                                           bool has_state, f4 (&O)[4], const h8 (&Qt)[2],
                                           const ChunkTmp& T)
{
    const int r = lane & 15, g = lane >> 4;
    const int t = 16 * w + r;
    f4 sc[4];
    if (!T.exact) {
        // Sc^T[s][t] = sum_i Kh[s][i] Qh[t][i] for s-blocks up to the diagonal
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) {
            sc[sb] = f4{0.f, 0.f, 0.f, 0.f};
            if (sb <= w) {
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    sc[sb] = mfma(ld8(sm.Kh, 16 * sb + r, 32 * ks + 8 * g), T.qh[ks], sc[sb]);
            }
        }
    } else {
        exact_scores(sm, R, T.x, w, lane, sc);
    }
    // mask, and write the wave's score rows Sc[t][s] (zeros above the diagonal)
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        h4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            hv[e] = (_Float16)((16 * sb + 4 * g + e <= t) ? sc[sb][e] : 0.f);
        st4(sm.Sc, t, 16 * sb + 4 * g, hv);
    }
    const int kmax = (w >= 2) ? 2 : 1;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
            if (ks < kmax)
                O[jt] = mfma(ld8(sm.VT, 16 * jt + r, 32 * ks + 8 * g), ld8(sm.Sc, t, 32 * ks + 8 * g),
                             O[jt]);
        if (has_state) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                O[jt] = mfma(ld8(st_tile(sm, st), 16 * jt + r, 32 * ks + 8 * g), Qt[ks], O[jt]);
        }
    }
}

// Store O (C layout, rows t = 16w + r) scaled, staged through the wave's rows of Sc.
__device__ __forceinline__ void store_out(Smem& sm, const FusedArgs& a, int b, int h, int t0, int w,
                                          int lane, const f4 (&O)[4])
{
    const int r = lane & 15, g = lane >> 4;
    const int t = 16 * w + r;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) st4(sm.Sc, t, 16 * jt + 4 * g, pack4(O[jt], a.scale));
    __builtin_amdgcn_wave_barrier();
    const long long off = row_offset(a, b, h, t0 + t);
    if (off >= 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const h8 val = ld8(sm.Sc, t, 8 * g + 32 * hh);
            __builtin_nontemporal_store(__builtin_bit_cast(u4, val),
                                        reinterpret_cast<u4*>(a.out + off + 8 * g + 32 * hh));
        }
    }
}

// Publish a span summary: U = local final state (C layout in S), D = decay
// of the span, as tagged words (U at i * 64 + j, D at 4096 + i).
__device__ __forceinline__ void publish_summary(const FusedArgs& a, const Smem& sm, const f4 (&S)[4],
                                                long long slot, int w, int lane)
{
    const int r = lane & 15, g = lane >> 4;
    const unsigned int tag = sm.tag;
    u64* my_agg = a.agg + slot * kAggWords;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            ll_store(my_agg + (16 * w + 4 * g + e) * kD + 16 * jt + r, S[jt][e], tag);
    if (w == 0) ll_store(my_agg + kD * kD + lane, ex2(sm.Pend[lane]), tag);
}

// ---------------------------------------------------------------------------
template <int SPAN, bool KEEP>
__global__ void __launch_bounds__(kThreads, (KEEP && SPAN == 1) ? 3 : 2)
gla_fused_kernel(FusedArgs a)
{
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;

    const int local_seq = blockIdx.x / a.n_spans;
    const int j = blockIdx.x - local_seq * a.n_spans;
    const int seq = a.seq0 + local_seq;
    const int b = seq / a.H, h = seq - (seq / a.H) * a.H;
    const int span = KEEP ? SPAN : a.span;
    const int c_first = j * span;
    const int n_c = min(span, a.n_chunks - c_first);

    ChunkRegs cur, nxt;
    load_chunk<KEEP>(a, b, h, c_first * kC, w, lane, cur);
    if (tid < kD) {
        sm.P[0][tid] = 0.f;
        sm.Pend[tid] = 0.f;
    }
    if (tid == 0) {
        sm.tag = __hip_atomic_load(a.epoch + local_seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    }

    // ---- 1. local pass --------------------------------------------------------
    // The span summary is published right after the last chunk's state update,
    // before that chunk's outputs, so the exchange overlaps them.
    const long long seq_slot = (long long)local_seq * a.n_spans;
    f4 S[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) S[n] = f4{0.f, 0.f, 0.f, 0.f};
    f4 O[KEEP ? SPAN : 1][4];
    h8 Qt[KEEP ? SPAN : 1][2];
    if (KEEP) {
#pragma unroll
        for (int c = 0; c < SPAN; ++c) {
#pragma unroll
            for (int n = 0; n < 4; ++n) O[c][n] = f4{0.f, 0.f, 0.f, 0.f};
            if (c < n_c) {
                if (c + 1 < n_c) load_chunk<true>(a, b, h, (c_first + c + 1) * kC, w, lane, nxt);
                ChunkTmp T;
                chunk_front<true>(sm, cur, w, lane, c, S, c & 1, c + 1 < n_c, Qt[c], T);
                if (c + 1 == n_c) publish_summary(a, sm, S, seq_slot + j, w, lane);
                chunk_back(sm, cur, w, lane, c & 1, c > 0, O[c], Qt[c], T);
                if (c + 1 < n_c) cur = nxt;
            }
        }
    } else {
        h8 qdummy[2];
        ChunkTmp T;
        for (int c = 0; c < n_c; ++c) {
            if (c + 1 < n_c) load_chunk<false>(a, b, h, (c_first + c + 1) * kC, w, lane, nxt);
            chunk_front<false>(sm, cur, w, lane, c, S, 0, false, qdummy, T);
            if (c + 1 < n_c) cur = nxt;
        }
        publish_summary(a, sm, S, seq_slot + j, w, lane);
    }

    // ---- 2. boundary scan across the sequence's spans -------------------------
    // Exchange words are indexed i * 64 + j (state row i, column j); the span
    // decays follow at 4096 + i.
    const unsigned int tag = sm.tag;
    lds_barrier();   // every wave is done with the chunk tiles
    // The chunk tiles are free now: 48 KB of LDS scratch for the exchange.
    unsigned char* scr = reinterpret_cast<unsigned char*>(sm.Kh);
    {
        // My slice: elements [e_first, e_first + ecount) of the state, through
        // every span of the sequence. All words arrive by DMA into LDS, tags
        // are checked there.
        const int ns = a.n_spans;
        const int e_first = j * a.slice;
        const int ecount = max(0, min(a.slice, kD * kD - e_first));
        if (ecount > 0) {
            const u64* agg0 = a.agg + seq_slot * kAggWords;
            u64* sin0 = a.sin + seq_slot * (kD * kD);
            const int i0 = e_first >> 6;
            const int nrows = ((e_first + ecount - 1) >> 6) - i0 + 1;
            u64* ubuf = reinterpret_cast<u64*>(scr);                 // [ns][ecount]
            float* dbuf = reinterpret_cast<float*>(scr + kScanU);    // [ns][nrows]
            float* compA = dbuf + kScanD;
            float* compB = compA + kThreads;
            const int half = ecount >> 1;              // 16 B lane loads per span
            const int nl = ns * half;
            for (unsigned int polls = 0;; ++polls) {
                for (int k0 = 64 * w; k0 < nl; k0 += kThreads) {
                    const int q = k0 + lane;
                    if (q < nl) {
                        const int m = q / half, pr = q - (q / half) * half;
                        __builtin_amdgcn_global_load_lds(
                            agg0 + (long long)m * kAggWords + e_first + 2 * pr, ubuf + 2 * k0, 16, 0,
                            kDevScope);
                    }
                }
                bool ok = true;
                for (int q = tid; q < ns * nrows; q += kThreads) {
                    const int m = q / nrows, rr = q - (q / nrows) * nrows;
                    float v;
                    ok &= ll_load(agg0 + (long long)m * kAggWords + kD * kD + i0 + rr, tag, v);
                    dbuf[q] = v;
                }
                __builtin_amdgcn_s_waitcnt(0x0F70);
                if (tid == 0) sm.stale = 0;
                lds_barrier();
                for (int q = tid; q < ns * ecount; q += kThreads)
                    ok &= (unsigned int)(ubuf[q] >> 32) == tag;
                if (!__all(ok) && lane == 0) sm.stale = 1;
                lds_barrier();
                const bool stale = sm.stale;
                if (!stale) break;
                if (polls > kMaxPolls) {
                    if (tid == 0) atomicOr(a.err, 1u);
                    break;
                }
                lds_barrier();   // every thread has read the flag before it is reset
                __builtin_amdgcn_s_sleep(2);
            }
            // P threads per element fold contiguous span ranges; LDS combines them
            int P = 1;
            while (P < 16 && ecount * P * 2 <= kThreads) P *= 2;
            const int epad = kThreads / P;
            const int p = tid / epad, el0 = tid - (tid / epad) * epad;
            const int per = (ns + P - 1) / P;
            const int m_lo = min(p * per, ns), m_hi = min(m_lo + per, ns);
            for (int eg = 0; eg < ecount; eg += epad) {
                const int el = eg + el0;
                const bool mine = el < ecount;
                const int elc = mine ? el : 0;
                const int e = e_first + elc;
                const int ir = (e >> 6) - i0;
                float A = 1.f, Bv = 0.f;
                for (int m = m_lo; m < m_hi; ++m) {
                    const float d = dbuf[m * nrows + ir];
                    A *= d;
                    Bv = d * Bv + __uint_as_float((unsigned int)ubuf[m * ecount + elc]);
                }
                compA[tid] = A;
                compB[tid] = Bv;
                lds_barrier();
                float run = 0.f;
                for (int pp = 0; pp < p; ++pp)
                    run = compA[pp * epad + el0] * run + compB[pp * epad + el0];
                if (mine) {
                    for (int m = m_lo; m < m_hi; ++m) {
                        ll_store(sin0 + (long long)m * (kD * kD) + e, run, tag);
                        run = dbuf[m * nrows + ir] * run +
                              __uint_as_float((unsigned int)ubuf[m * ecount + elc]);
                    }
                    if (p == P - 1 && a.final_state)
                        a.final_state[(long long)seq * kD * kD + e] = run;
                }
                lds_barrier();   // comp reusable
            }
        }
        lds_barrier();   // scratch free again
    }

    // my incoming state S_in (C layout), by DMA into the scratch
    f4 Sin[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) Sin[n] = f4{0.f, 0.f, 0.f, 0.f};
    if (j > 0) {
        const u64* src = a.sin + (seq_slot + j) * (kD * kD);
        u64* sbuf = reinterpret_cast<u64*>(scr);
        for (unsigned int polls = 0;; ++polls) {
#pragma unroll
            for (int k0 = 0; k0 < kD * kD / 2; k0 += kThreads)
                __builtin_amdgcn_global_load_lds(src + 2 * (k0 + 64 * w + lane), sbuf + 2 * (k0 + 64 * w),
                                                 16, 0, kDevScope);
            __builtin_amdgcn_s_waitcnt(0x0F70);
            if (tid == 0) sm.stale = 0;
            lds_barrier();
            bool ok = true;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u64 x = sbuf[(16 * w + 4 * g + e) * kD + 16 * jt + r];
                    ok &= (unsigned int)(x >> 32) == tag;
                    Sin[jt][e] = __uint_as_float((unsigned int)x);
                }
            if (!__all(ok) && lane == 0) sm.stale = 1;
            lds_barrier();
            const bool stale = sm.stale;
            if (!stale) break;
            if (polls > kMaxPolls) {
                if (tid == 0) atomicOr(a.err, 1u);
                break;
            }
            lds_barrier();   // every thread has read the flag before it is reset
            __builtin_amdgcn_s_sleep(2);
        }
    }
    // Every slice owner has read every span's summary before the last span's
    // S_in is complete, so every workgroup of the sequence has read this
    // launch's tag by then: advance it for the next launch.
    if (j == a.n_spans - 1 && tid == 0)
        __hip_atomic_store(a.epoch + local_seq, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    // ---- 3. outputs -----------------------------------------------------------
    if (KEEP) {
        if (j > 0) {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                st4(sm.ST0, 16 * jt + r, 16 * w + 4 * g, pack4(Sin[jt], 1.f));
        }
        lds_barrier();
#pragma unroll
        for (int c = 0; c < SPAN; ++c) {
            if (c >= n_c) continue;
            if (j > 0) {
                // q 2^b scaled by the decay from the span start to this chunk
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    h8 qs = Qt[c][hh];
                    if (c > 0) {
                        float p[8];
                        ld_f8(&sm.P[c][32 * hh + 8 * g], p);
#pragma unroll
                        for (int e = 0; e < 8; ++e) qs[e] = (_Float16)((float)qs[e] * ex2(p[e]));
                    }
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt)
                        O[c][jt] = mfma(ld8(sm.ST0, 16 * jt + r, 32 * hh + 8 * g), qs, O[c][jt]);
                }
            }
            store_out(sm, a, b, h, (c_first + c) * kC, w, lane, O[c]);
        }
    } else {
        // stream the span again from its incoming state
#pragma unroll
        for (int n = 0; n < 4; ++n) S[n] = Sin[n];
        if (j > 0) {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                st4(sm.ST0, 16 * jt + r, 16 * w + 4 * g, pack4(S[jt], 1.f));
        }
        load_chunk<true>(a, b, h, c_first * kC, w, lane, cur);
        int st = 0;
        for (int c = 0; c < n_c; ++c) {
            if (c + 1 < n_c) load_chunk<true>(a, b, h, (c_first + c + 1) * kC, w, lane, nxt);
            f4 Oc[4];
            h8 qt[2];
#pragma unroll
            for (int n = 0; n < 4; ++n) Oc[n] = f4{0.f, 0.f, 0.f, 0.f};
            ChunkTmp T;
            chunk_front<true>(sm, cur, w, lane, kMaxKeep, S, st, c + 1 < n_c, qt, T);
            chunk_back(sm, cur, w, lane, st, (j > 0) || (c > 0), Oc, qt, T);
            store_out(sm, a, b, h, (c_first + c) * kC, w, lane, Oc);
            st ^= 1;
            if (c + 1 < n_c) cur = nxt;
        }
    }
}

// ---------------------------------------------------------------------------
bool fused_supported(const Shape& s)
{
    return s.d_k == kD && s.d_v == kD && s.chunk == kC;
}

static int device_cus()
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

static const void* pick_kernel(int span, bool keep)
{
    if (!keep) return (const void*)gla_fused_kernel<1, false>;
    if (span == 1) return (const void*)gla_fused_kernel<1, true>;
    return (const void*)gla_fused_kernel<2, true>;
}

// Dynamic LDS of a variant: one-chunk spans never touch the second state buffer.
static size_t smem_bytes(int span, bool keep)
{
    return (keep && span == 1) ? offsetof(Smem, ST1) : sizeof(Smem);
}

// Workgroups of one variant that fit on a CU at once.
static int resident_per_cu(int span, bool keep)
{
    static int cache[2][kMaxKeep + 1] = {};
    int& c = cache[keep ? 1 : 0][keep ? span : 0];
    if (c == 0) {
        const void* fn = pick_kernel(span, keep);
        int n = 0;
        const size_t sh = smem_bytes(span, keep);
        if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh) !=
                hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, sh) != hipSuccess ||
            n < 1)
            n = 1;
        c = n;
    }
    return c;
}

FusedPlan fused_plan(const Shape& s, int span_override)
{
    FusedPlan p;
    const int n_seq = s.B * s.H;
    const int nc = s.n_chunks;
    auto fill = [&](int span, bool keep) {
        p.span = span;
        p.keep = keep;
        p.n_spans = (nc + span - 1) / span;
        const long long cap = (long long)resident_per_cu(span, keep) * device_cus();
        // sequences per launch, so that every workgroup of a launch is resident
        long long per = cap / p.n_spans;
        if (per < 1) per = 1;
        p.seq_batch = (int)(per < n_seq ? per : n_seq);
        p.grid = p.seq_batch * p.n_spans;
        p.slice = 16 * ((256 + p.n_spans - 1) / p.n_spans);
    };
    auto one_seq_fits = [&]() {
        return (long long)p.n_spans <= (long long)resident_per_cu(p.span, p.keep) * device_cus();
    };
    if (span_override > 0) {
        fill(span_override, span_override <= kMaxKeep);
        while (!one_seq_fits() || p.n_spans > kMaxSpans) fill(p.span * 2, false);
        return p;
    }
    // the shortest kept span whose whole grid is resident; else streamed spans
    for (int sp = 1; sp <= kMaxKeep; ++sp) {
        fill(sp, true);
        if (p.seq_batch == n_seq && p.n_spans <= kMaxSpans) return p;
    }
    const long long cap = (long long)resident_per_cu(1, false) * device_cus();
    long long per_seq = cap / n_seq;
    if (per_seq < 1) per_seq = 1;
    if (per_seq > kMaxSpans) per_seq = kMaxSpans;
    fill((int)((nc + per_seq - 1) / per_seq), false);
    while (!one_seq_fits() || p.n_spans > kMaxSpans) fill(p.span * 2, false);
    return p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

size_t fused_workspace_bytes(const Shape& s, const FusedPlan& p)
{
    (void)s;
    const size_t nb = (size_t)p.seq_batch;
    return 256 + align256(nb * sizeof(unsigned int)) +
           nb * p.n_spans * (size_t)(kAggWords + kD * kD) * sizeof(u64);
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const void* lg,
                        const Shape& s, const FusedPlan& p, void* out, float* final_state,
                        void* ws, hipStream_t st)
{
    FusedArgs a;
    a.q = (const __half*)q;
    a.k = (const __half*)k;
    a.v = (const __half*)v;
    a.lg = (const __half*)lg;
    a.out = (__half*)out;
    a.final_state = final_state;
    unsigned char* base = (unsigned char*)ws;
    const size_t nb = (size_t)p.seq_batch;
    a.err = (unsigned int*)base;
    a.epoch = (unsigned int*)(base + 256);
    a.agg = (u64*)(base + 256 + align256(nb * sizeof(unsigned int)));
    a.sin = a.agg + nb * p.n_spans * kAggWords;
    a.L = s.L;
    a.H = s.H;
    a.grid_h = s.grid_h;
    a.grid_w = s.grid_w;
    a.dir = s.dir;
    a.n_chunks = s.n_chunks;
    a.span = p.span;
    a.n_spans = p.n_spans;
    a.slice = p.slice;
    a.scale = s.scale;
    const void* fn = pick_kernel(p.span, p.keep);
    resident_per_cu(p.span, p.keep);   // also raises the kernel's dynamic LDS limit
    const int n_seq = s.B * s.H;
    for (int s0 = 0; s0 < n_seq; s0 += p.seq_batch) {
        a.seq0 = s0;
        const int nseq = (n_seq - s0 < p.seq_batch) ? (n_seq - s0) : p.seq_batch;
        void* args[] = {&a};
        const hipError_t e = hipLaunchKernel(fn, dim3(nseq * p.n_spans), dim3(kThreads), args,
                                             smem_bytes(p.span, p.keep), st);
        if (e != hipSuccess) return e;
    }
    return hipGetLastError();
}

}  // namespace gtrgla
