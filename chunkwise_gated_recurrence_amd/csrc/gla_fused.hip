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
// Exchanged values travel as 4-byte words: an fp32 value rounded to 16
// mantissa bits whose low 8 bits carry a tag (span summaries), or as 2-byte
// fp16 words whose lowest mantissa bit carries the tag's parity (incoming
// states, which the output pass uses in fp16), written and read with
// device-scope (sc1) accesses. A reader polls the words themselves until every
// tag equals the expected one, so a hand-over costs one memory round trip: no
// flags, no fences, no atomics. Each exchange slot (sequence in the launch,
// span) has its own epoch in the workspace; the words of a slot are rewritten
// in full by every launch that uses it and its epoch is advanced once all of
// that launch's readers know it, so the words in memory always carry the
// previous tag and a workspace is cleared only once. The rounding perturbs a
// summary value by at most 2^-16 of itself and an incoming state by at most
// 2^-10 (fp16 with its last bit taken; the final state is folded from the
// summaries in fp32).
//
// One counter tracks a wave's loads and stores together, so a wave that waits
// for a load also waits for every store it has in flight: the span summary is
// stored by waves 2-3 only, which keeps its store latency off waves 0-1's
// first polls. The owners' fold stores the incoming states straight from the
// fold (all waves), and each wave then polls its own rows of its incoming
// state.
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
#include <atomic>
#include <cstdlib>
#include <type_traits>

#include "gla_common.h"
#include "gla_launch.h"
#include "gla_ws.h"

namespace gtrgla {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef unsigned long long u64;

constexpr int kC = 64;            // chunk length
constexpr int kD = 64;            // d_k = d_v
constexpr int kThreads = 256;     // 4 waves
constexpr int kMaxKeep = 8;       // longest span kept on chip
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kGuard = 16.0f;   // max log2 range of a chunk for factorised scores
constexpr int kTile = kC * 72;    // halves per LDS tile (rows padded to 72)
constexpr int kAggWords = kD * kD + kD;   // U and D words of one span summary
constexpr int kMaxSpans = 64;        // spans per sequence
constexpr int kScanD = 32 * 1024;    // exchange scratch: byte offset of the decays
constexpr int kDevScope = 16;        // cache policy: device-scope (sc1) access
constexpr int kSinSlotBytes = kD * kD * 2;   // incoming-state words of one span slot (2 B each)
constexpr int kPollSleep = 2;        // s_sleep between incoming-state polls (64 clocks each)

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

// Tagged exchange words: value rounded to nearest at 16 mantissa bits, tag in
// the low 8 bits.
__device__ __forceinline__ unsigned int ll_word(float v, unsigned int tag)
{
    return ((__float_as_uint(v) + 0x80u) & 0xFFFFFF00u) | tag;
}
__device__ __forceinline__ float ll_value(unsigned int x) { return __uint_as_float(x & 0xFFFFFF00u); }
__device__ __forceinline__ bool ll_ok(unsigned int x, unsigned int tag) { return (x & 0xFFu) == tag; }

// Incoming-state words are 2 bytes: the value in fp16 (the output pass uses
// the incoming state in fp16) with its lowest mantissa bit replaced by the
// parity of the tag. The parity suffices: every launch that uses a slot
// rewrites all of its words and advances its epoch by one, so a stale word
// always carries the previous launch's tag.
__device__ __forceinline__ unsigned short sin_word(float v, unsigned int tag)
{
    const unsigned short x = __builtin_bit_cast(unsigned short, (_Float16)v);
    return (unsigned short)((x & 0xFFFEu) | (tag & 1u));
}
__device__ __forceinline__ bool sin_ok(unsigned short x, unsigned int tag) { return ((x ^ tag) & 1u) == 0; }
// (the tag bit is cleared, so that the value does not depend on the launch)
__device__ __forceinline__ float sin_value(unsigned short x)
{
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(x & 0xFFFEu));
}

// Buffer resource over n_bytes at base: accesses past the end read zeros and
// are dropped on write.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int n_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n_bytes, 0x00020000);
}
__device__ __forceinline__ void st_dev1(__amdgpu_buffer_rsrc_t rs, int voff, unsigned int x)
{
    __builtin_amdgcn_raw_buffer_store_b32(x, rs, voff, 0, kDevScope);
}
__device__ __forceinline__ void st_dev4(__amdgpu_buffer_rsrc_t rs, int voff, u4 x)
{
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, voff, 0, kDevScope);
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
// Lane (n, kb) holds B[8kb .. 8kb+7][n]: at most one 1.0 (fp16 0x3C00), at
// element e = n + 16 half - 8 kb when that is in 0..7.
__device__ __forceinline__ h8 selector(int lane, int half)
{
    const int e = (lane & 15) + 16 * half - 8 * (lane >> 4);
    const unsigned int one = 0x3C00u << (16 * (e & 1));
    u4 u;
#pragma unroll
    for (int d = 0; d < 4; ++d) u[d] = (e >> 1) == d ? one : 0u;
    return __builtin_bit_cast(h8, u);
}

// ---------------------------------------------------------------------------
struct FusedArgs {
    const __half* q;
    const __half* k;
    const __half* v;
    const __half* lg;
    __half* out;
    float* final_state;
    unsigned int* epoch;        // [seq in launch][n_spans] low 8 bits: tag of the slot's words
    unsigned int* hdr;          // workspace header (gla_ws.h): error word, magic, layout
    unsigned int* agg;          // [seq in launch][agg_seq_words(n_spans)]  tagged, owner-major
    unsigned int* sin;          // [seq in launch][n_spans] slots of kSinSlotBytes: 2-byte words
    u4* park;                   // [workgroup][span - 1][256 threads][4]: parked outputs (long kept spans)
    int L, H, grid_h, grid_w, dir;
    int n_chunks;               // per sequence
    int span;                   // chunks per workgroup
    int n_spans;                // workgroups per sequence
    int seq0;                   // first sequence of this launch
    int slice_log2;             // log2 of the state elements each owner scans
    int dk;                     // key dim of q, k, log_gamma: 64, or 32 (zero-padded to 64 on load)
    float scale;
    const float* init;          // [B, H, 64, 64] states before the first step, or null (zero)
    const __half* gate;         // [B, L, H, 64] output gate, or null (outputs as they are)
    const float* norm_w;        // [64] RMSNorm weight of the output epilogue (with gate)
    float eps;
    // log_gamma computed in the kernel from the low-rank gate (else read from lg):
    // lg = inv_tau * logsigmoid(z W2 + bias), z = x W1 per token
    const float* z;             // [B, L, 16] x W1
    const float* w2;            // [16, H * dk]
    const float* gbias;         // [H * dk]
    float inv_tau;
    int gtab_off;               // byte offset of the low-rank gate tables in dynamic LDS
    unsigned int layout;        // exchange layout word of this launch (header word 2)
    int fault;                  // test hook: nonzero, span 0 of every sequence publishes nothing
    unsigned long long wait_ticks;   // longest wait of one exchange poll loop (100 MHz ticks)
};

// Dynamic LDS of every fused kernel: its Smem (or SmemRK), then, for the
// low-rank gate, the W2 operand table and the bias.
extern __shared__ __align__(16) unsigned char smem_raw[];

// Low-rank gate tables: the A operand of the 16x16x32 fp16 MFMA that forms
// z W2 for tile jt (16 key dims), with the tile's rows (dims) permuted so that
// the product lands in the layout of the chunk operands (lane (r, g) of a
// wave: row r, dims 8g + e + 32hh); and the bias per key dim. W2 enters in two
// fp16 parts, hi = fp16(W2) and lo = fp16(W2 - hi): the K = 32 of the MFMA
// runs over (rank, part), lane (m, kb) holding ranks 8(kb & 1) .. + 7 of hi
// (kb < 2) or of lo (kb >= 2) for dim col(m, jt).
struct GateTab {
    h8 w2[4][64];       // [jt][lane]
    float bias[kD];
};
__device__ __forceinline__ int gate_col(int m, int jt)
{
    return 8 * (m >> 2) + 4 * (jt & 1) + (m & 3) + 32 * (jt >> 1);
}

// Fill head h's gate tables (every thread of the workgroup; the caller puts a
// barrier before their first use). Key dims past dk get zero weight and bias.
__device__ __forceinline__ void fill_gate_tables(const FusedArgs& a, int h, int tid)
{
    GateTab& gt = *reinterpret_cast<GateTab*>(smem_raw + a.gtab_off);
    const int K = a.H * a.dk;
    for (int q = tid; q < 4 * 64 * 8; q += kThreads) {
        const int e = q & 7, ln = (q >> 3) & 63, jt = q >> 9, kb = ln >> 4;
        const int col = gate_col(ln & 15, jt);
        const float v = col < a.dk ? a.w2[(8 * (kb & 1) + e) * K + h * a.dk + col] : 0.f;
        const _Float16 hi = (_Float16)v;
        reinterpret_cast<_Float16*>(&gt.w2[jt][ln])[e] = kb < 2 ? hi : (_Float16)(v - (float)hi);
    }
    if (tid < kD) gt.bias[tid] = tid < a.dk ? a.gbias[h * a.dk + tid] : 0.f;
}

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
    _Float16 cp16[kD];        // 2^{P_c}: decay from the span start to the chunk start
    float dcv[kD];            // 2^{b_last} = d_c
    float blast[kD];          // b_last (log2 of d_c)
    float P[kMaxKeep + 1][kD];  // log2 decay from the span start to each chunk start
    float Pend[kD];           // log2 decay of the span so far
    float nw[kD];             // RMSNorm weight of the output epilogue
    unsigned int tags[kMaxSpans];   // expected tag of every span slot of the sequence
    int fail;
    int stale;
    int dstale;   // exchange: a decay word was stale in this poll
    int expired;  // exchange: the owners' wait has passed its deadline
    int poison;   // exchange: this workgroup's incoming state is missing or NaN
    int wsbad;    // the workspace header does not allow this launch
    unsigned int hdr[4];   // the workspace header, staged by wave 0 at the start
};


struct ChunkRegs {
    u4 q[2], k[2], v[2], g[2];   // g: log_gamma, or (low-rank gate) the row's z
    bool valid;                  // low-rank gate: the row is a token of the sequence
};

// Row offset (halves) of scan step t of sequence (b, h); -1 past the end.
__device__ __forceinline__ long long row_offset(const FusedArgs& a, int b, int h, int t)
{
    if (t >= a.L) return -1;
    const int p = scan_to_spatial(t, a.L, a.grid_h, a.grid_w, a.dir);
    return (((long long)b * a.L + p) * a.H + h) * kD;
}

// Buffer resource over batch b of a [B, L, H, d] fp16 tensor. Buffer loads
// past num_records return zeros, so rows beyond the sequence end read as zero
// without a branch (a branch around a load makes the compiler wait for it).
constexpr int kNT = 0;   // cache policy of the chunk loads: default (a streaming hint measured slower)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t batch_rsrc(const __half* base, const FusedArgs& a,
                                                             int b, int d = kD)
{
    const long long per_batch = (long long)a.L * a.H * d;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + b * per_batch), (short)0,
                                             (int)(per_batch * 2), 0x00020000);
}

// Byte offsets of 16-byte block blk (dims 8 blk .. 8 blk + 7) of scan step t of
// head h: key side (q, k, log_gamma: rows of dk halves; blocks past dk read
// zeros, so a 32-wide key dim is zero-padded to 64) and value side (v: rows of
// 64 halves). Past the sequence end both read zeros.
struct RowOff {
    int key, val;
};
__device__ __forceinline__ RowOff row_off(const FusedArgs& a, int h, int t, int blk)
{
    const int kbytes = a.L * a.H * a.dk * 2, vbytes = a.L * a.H * kD * 2;
    if (t >= a.L) return RowOff{kbytes, vbytes};
    const int ph = scan_to_spatial(t, a.L, a.grid_h, a.grid_w, a.dir) * a.H + h;
    return RowOff{8 * blk < a.dk ? ph * (a.dk * 2) + 16 * blk : kbytes, ph * (kD * 2) + 16 * blk};
}

__device__ __forceinline__ u4 load16(__amdgpu_buffer_rsrc_t rs, int voff)
{
    return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, 0, kNT));
}

// Low-rank gate input of scan step t for lane l: z[8((l >> 4) & 1) .. +7] of
// the row (the B operand of the gate MFMAs); zeros past the sequence end.
__device__ __forceinline__ void load_z(const FusedArgs& a, int b, int t, int lane, u4 (&z)[2])
{
    const int bytes = a.L * 64;
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.z + (long long)b * a.L * 16), (short)0, bytes, 0x00020000);
    const int voff = t < a.L ? scan_to_spatial(t, a.L, a.grid_h, a.grid_w, a.dir) * 64 +
                                   32 * ((lane >> 4) & 1)
                             : bytes;
    z[0] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rz, voff, 0, kNT));
    z[1] = __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(rz, voff, 16, kNT));
}

// Lane l of wave w loads row 16w + (l & 15), dims 8(l >> 4) + 32h .. +7.
template <bool WITH_Q>
__device__ __forceinline__ void load_chunk(const FusedArgs& a, int b, int h, int t0, int w,
                                           int lane, ChunkRegs& R)
{
    const int t = t0 + 16 * w + (lane & 15);
    const __amdgpu_buffer_rsrc_t rk = batch_rsrc(a.k, a, b, a.dk), rv = batch_rsrc(a.v, a, b),
                                 rg = batch_rsrc(a.lg, a, b, a.dk);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const RowOff o = row_off(a, h, t, (lane >> 4) + 4 * hh);
        if (WITH_Q) R.q[hh] = load16(batch_rsrc(a.q, a, b, a.dk), o.key);
        R.k[hh] = load16(rk, o.key);
        R.v[hh] = load16(rv, o.val);
        if (!a.z) R.g[hh] = load16(rg, o.key);
    }
    if (a.z) {   // z, and whether the row is a token (rows past the end get no decay)
        load_z(a, b, t, lane, R.g);
        R.valid = t < a.L;
    }
}

// Exact fp32 scores of the wave's rows t = 16w + r for a chunk whose gate
// range is too wide for the factorised form. chunk_front has put the fp32
// prefix of every row in the Kh+Sc table; raw k goes to KtT (the state update
// has consumed it); each lane sums its own 16 dims and four lanes (one per dim
// group) combine.
__device__ void exact_scores(Smem& sm, const FusedArgs& a, int b, int h, int t0, int w, int lane,
                             f4 (&sc)[4])
{
    const int r = lane & 15, g = lane >> 4;
    const int t = 16 * w + r;
    float* Bt = reinterpret_cast<float*>(sm.Kh);       // [64][64] fp32, overlays Kh and Sc
    _Float16* Kr = sm.KtT;                             // [64][64] raw k, row-major
    // raw q and k of the chunk again (rare path; the chunk registers hold the
    // next chunk by now)
    ChunkRegs R;
    load_chunk<true>(a, b, h, t0, w, lane, R);
    lds_barrier();
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        *reinterpret_cast<u4*>(Kr + t * kD + 32 * hh + 8 * g) = R.k[hh];
    lds_barrier();
    float x[2][8];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) ld_f8(Bt + t * kD + 32 * hh + 8 * g, x[hh]);
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
    bool exact;      // exact scores: the log2 prefix of every row is in the Kh+Sc table
};

// Front half of one chunk: log2-gate prefix, per-dim constants, operand tiles,
// and the state update S <- Diag(d_c) S + (k 2^{b_last-b})^T v. S (C layout:
// rows 16w+4g+e, cols 16jt+r) enters as the state at the chunk start and
// leaves as the state after it; the entering state is staged transposed in
// ST0 when stage_state. FULL also prepares the output half (Qt = q 2^b, Kh,
// qh). after_a runs right after the first barrier, when every wave has taken
// its operands out of R's source.
struct NoHook {
    __device__ void operator()() const {}
};

// log_gamma of the lane's chunk operands (row r, dims 8g + e + 32hh) from the
// low-rank gate: per dim tile, two 16x16x32 fp16 MFMAs of the W2 table with z
// (z_hi twice, for W2_hi and W2_lo; then z_lo for W2_hi: the dropped
// W2_lo z_lo is about 2^-22 of the product), the bias as the accumulator's
// start, then inv_tau * logsigmoid. z holds the lane's ranks 8(g & 1) .. + 7.
// A 32-wide key dim leaves dims 32..63 zero, and so does a row past the
// sequence end (valid false: gamma = 1 there, as the zero log_gamma that a
// read past the end gives on the other path).
__device__ __forceinline__ void lowrank_gate(const FusedArgs& a, const u4 (&z)[2], bool valid,
                                             int lane, float (&x)[2][8])
{
    const GateTab& gt = *reinterpret_cast<const GateTab*>(smem_raw + a.gtab_off);
    const int g = lane >> 4;
    h8 bh, bl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = __uint_as_float(z[e >> 2][e & 3]);
        const _Float16 hi = (_Float16)v;
        bh[e] = hi;
        bl[e] = g < 2 ? (_Float16)(v - (float)hi) : (_Float16)0.f;
    }
    const float sc = valid ? a.inv_tau : 0.f;
    // dims 32hh .. 32hh + 31: tiles 2hh and 2hh + 1
    auto half = [&](int hh) {
        f4 acc[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int jt = 2 * hh + j;
            acc[j] = *reinterpret_cast<const f4*>(&gt.bias[8 * g + 4 * j + 32 * hh]);
            const h8 wa = gt.w2[jt][lane];
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, bh, acc[j], 0, 0, 0);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wa, bl, acc[j], 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float y = acc[j][e];
                // log sigma(y) = min(y, 0) - ln(1 + e^{-|y|})
                const float ls = fminf(y, 0.f) -
                                 0.69314718f * __builtin_amdgcn_logf(1.f + ex2(-kLog2e * fabsf(y)));
                x[hh][4 * j + e] = sc * ls;
            }
        }
    };
    half(0);
    if (a.dk > 32) {
        half(1);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[1][e] = 0.f;
    }
}

template <bool FULL, class AfterA = NoHook>
__device__ __forceinline__ void chunk_front(const FusedArgs& a, Smem& sm, const ChunkRegs& R, int w,
                                            int lane, int c,
                                            f4 (&S)[4], bool stage_state, h8 (&Qt)[2], ChunkTmp& T,
                                            AfterA after_a = AfterA{})
{
    const int r = lane & 15, g = lane >> 4;
    const int tid = 64 * w + lane;

    // -- log2 gates, inclusive prefix over the wave's 16 rows
    float x[2][8];
    if (a.z) {
        lowrank_gate(a, R.g, R.valid, lane, x);
    } else {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) unpack8(R.g[hh], x[hh]);
    }
    // step-major, so that consecutive DPP adds are independent (a DPP read
    // of a value written by the previous instruction needs wait states)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[hh][e] *= kLog2e;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[hh][e] += row_shr<1>(x[hh][e]);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[hh][e] += row_shr<2>(x[hh][e]);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[hh][e] += row_shr<4>(x[hh][e]);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) x[hh][e] += row_shr<8>(x[hh][e]);
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
    after_a();      // every wave has read its chunk operands by now
    // the state entering this chunk, for its outputs (ST0 is free: the
    // previous chunk's output half has passed barrier A)
    if (stage_state) {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
            st4(sm.ST0, 16 * jt + r, 16 * w + 4 * g, pack4(S[jt], 1.f));
    }

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
        sm.cp16[d] = (_Float16)ex2(sm.P[c][d]);
        if (c < kMaxKeep) sm.P[c + 1][d] = sm.P[c][d] + bl;
        const bool wide = __any((bf - bl) > kGuard);
        if (d == 0) sm.fail = wide ? 1 : 0;
    }
    lds_barrier();  // (A2)

    // every per-dim constant of the lane's dims at once (one LDS round trip)
    const bool exact = FULL && sm.fail;
    float pre_c[2][8], ref_c[2][8];
    h8 cq_c[2], ck_c[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int d0 = 32 * hh + 8 * g;
        ld_f8(&sm.pre[w][d0], pre_c[hh]);
        if (FULL) {
            ld_f8(&sm.ref[d0], ref_c[hh]);
            cq_c[hh] = *reinterpret_cast<const h8*>(&sm.cq16[d0]);
            ck_c[hh] = *reinterpret_cast<const h8*>(&sm.ck16[d0]);
        }
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
        const int d0 = 32 * hh + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[hh][e] += pre_c[hh][e];
        h8 kt8;
        if (FULL && !exact) {
            // E = 2^{b-r} and 1/E in fp32, the products in packed fp16
            float ef[8], ei[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float dlt = x[hh][e] - ref_c[hh][e];
                ef[e] = ex2(dlt);
                ei[e] = ex2(-dlt);
            }
            const h8 cq = cq_c[hh];
            const h8 ck = ck_c[hh];
            const h8 q8 = __builtin_bit_cast(h8, R.q[hh]);
            const h8 k8 = __builtin_bit_cast(h8, R.k[hh]);
            const h8 qh = q8 * pack8(ef);
            const h8 kh = k8 * pack8(ei);
            T.qh[hh] = qh;
            Qt[hh] = qh * cq;
            kt8 = kh * ck;
            st8(sm.Kh, 16 * w + r, d0, kh);
        } else {
            if (exact) {   // the prefix table of the exact scores (Kh is unused then)
                float* Bt = reinterpret_cast<float*>(sm.Kh);
                *reinterpret_cast<f4*>(Bt + (16 * w + r) * kD + d0) = f4{x[hh][0], x[hh][1], x[hh][2], x[hh][3]};
                *reinterpret_cast<f4*>(Bt + (16 * w + r) * kD + d0 + 4) = f4{x[hh][4], x[hh][5], x[hh][6], x[hh][7]};
            }
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
    if (FULL) T.exact = exact;
}

// Output half of one chunk: O^T[j][t] += sum_s VT[j][s] Sc[t][s], plus
// sum_i ST0[j][i] Qt[t][i] when has_state.
__device__ __forceinline__ void chunk_back(Smem& sm, const FusedArgs& a, int b, int h, int t0, int w,
                                           int lane, bool has_state, f4 (&O)[4], const h8 (&Qt)[2],
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
        exact_scores(sm, a, b, h, t0, w, lane, sc);
    }
    // mask, and write the wave's score rows Sc[t][s] (zeros above the
    // diagonal): blocks left of the wave's diagonal block are whole, blocks
    // right of it are zero (w is uniform, so these are scalar branches)
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
        h4 hv;
        if (sb < w) {
            hv = pack4(sc[sb], 1.f);
        } else if (sb == w) {
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = (_Float16)((4 * g + e <= r) ? sc[sb][e] : 0.f);
        } else {
            hv = h4{0, 0, 0, 0};
        }
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
                O[jt] = mfma(ld8(sm.ST0, 16 * jt + r, 32 * ks + 8 * g), Qt[ks], O[jt]);
        }
    }
}

// Gate of a chunk's rows for the output epilogue, in store_out's layout (lane
// (r, g) of wave w: row 16w + r, dims 8g + 32hh .. +7). No gate: zeros, no
// memory access (an empty buffer resource).
__device__ __forceinline__ void load_gate(const FusedArgs& a, int b, int h, int t0, int w, int lane,
                                          u4 (&z)[2])
{
    const int t = t0 + 16 * w + (lane & 15);
    const long long per_batch = (long long)a.L * a.H * kD;
    const int bytes = a.gate ? (int)(per_batch * 2) : 0;
    const int voff = t < a.L
        ? (scan_to_spatial(t, a.L, a.grid_h, a.grid_w, a.dir) * a.H + h) * (kD * 2) + 16 * (lane >> 4)
        : (int)(per_batch * 2);
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.gate + (a.gate ? b * per_batch : 0)), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) z[hh] = load16(rz, voff + 64 * hh);
}

// Store O (C layout, rows t = 16w + r) scaled, staged through the wave's rows
// of Sc. With a gate, the output epilogue: each row o (scaled) becomes
// o / sqrt(mean(o^2) + eps) * w * SiLU(z), z from load_gate (the row's mean
// square is summed over the four lanes that hold it).
__device__ __forceinline__ void store_out(Smem& sm, const FusedArgs& a, int b, int h, int t0, int w,
                                          int lane, const f4 (&O)[4], const u4 (&z)[2],
                                          bool poison = false)
{
    const int r = lane & 15, g = lane >> 4;
    const int t = 16 * w + r;
    float f = a.scale;
    if (a.gate) {
        float ss = 0.f;
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += O[jt][e] * O[jt][e];
        ss += __shfl_xor(ss, 16, 64);
        ss += __shfl_xor(ss, 32, 64);
        f = a.scale * __builtin_amdgcn_rsqf(a.scale * a.scale * ss * (1.f / kD) + a.eps);
    }
    if (poison) f = __builtin_nanf("");   // the failure path: every output NaN
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) st4(sm.Sc, t, 16 * jt + 4 * g, pack4(O[jt], f));
    __builtin_amdgcn_wave_barrier();
    const long long off = row_offset(a, b, h, t0 + t);
    if (off >= 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            h8 val = ld8(sm.Sc, t, 8 * g + 32 * hh);
            if (a.gate) {
                float zf[8], wf[8];
                unpack8(z[hh], zf);
                ld_f8(&sm.nw[8 * g + 32 * hh], wf);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    val[e] = (_Float16)((float)val[e] * wf[e] * zf[e] *
                                        rcp(1.f + ex2(-kLog2e * zf[e])));
            }
            __builtin_nontemporal_store(__builtin_bit_cast(u4, val),
                                        reinterpret_cast<u4*>(a.out + off + 8 * g + 32 * hh));
        }
    }
}

// ---- workspace header (gla_ws.h)
// The header, staged in LDS by wave 0 at the start (a 4-byte DMA per lane of
// lanes 0-3, device scope): no registers are held for it, and wave 0's wait
// for its chunk loads (issued after it) also covers it.
__device__ __forceinline__ void stage_ws_header(const FusedArgs& a, unsigned int* hdr_lds, int w,
                                                int lane)
{
    if (w == 0 && lane < 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc(a.hdr, kWsHeaderBytes),
                                                 (__attribute__((address_space(3))) void*)hdr_lds,
                                                 4, 4 * lane, 0, 0, kDevScope);
}
// Whether this launch may use the workspace's exchange words: no error since
// the last status check, and the region either zeroed by the library or last
// used by fused launches of this very layout.
__device__ __forceinline__ bool ws_header_ok(const FusedArgs& a, const unsigned int* hv)
{
    const unsigned int magic = hv[kWsMagicWord];
    return hv[kWsErrWord] == 0 &&
           (magic == kWsClean ||
            (magic == kWsFused && hv[kWsLayoutWord] == a.layout && hv[kWsLayoutCheck] == ~a.layout));
}
// Summary words of one sequence, owner-major: for each owner o (slice of
// 2^lo state elements) a contiguous region [ns][slice] of U words, then
// [ns][slice / 64] D words (the decays of the slice's state rows), padded to
// 16 bytes. An owner then reads its whole input as one contiguous block.
__device__ __forceinline__ int owner_region_words(int ns, int lo)
{
    return (ns << lo) + (((ns << (lo - 6)) + 3) & ~3);
}
__host__ __device__ inline long long agg_seq_words(int ns) { return (long long)ns * kAggWords + 256; }

// Publish a span summary: U = local final state (C layout in S), D = decay
// of the span, as tagged words of slot `slot` (U at i * 64 + j, D at 4096 + i).
// Also turns the epochs loaded at the start (thread t < n_spans holds the one
// of span t in ep) into the tag table. Waves 0-1 hand their U rows to the
// storer waves through an LDS tile that the chunk's output half does not read:
// ST0 when that half takes no incoming state (AFTER_STATE false), else KtT,
// after a barrier (every wave's state update has read its KtT rows by then).
// Two waves store because a wave's wait for a load also waits for its own
// earlier stores, and device-scope stores are acknowledged late: storing from
// every wave made the exchange's first polls return about 1 us later.
constexpr int kU01 = 68;   // fp32 row stride of the handed-over rows (no bank conflicts)

// u23: an LDS region of 32 rows x kU01 floats that no later read of the chunk
// needs (or null): waves 2-3 then stage their rows too, and every row goes
// out in 16-byte stores (fewer, wider stores than one word per lane). The
// one-chunk kernel passes ST0 (with KtT as u01 after the AFTER_STATE
// barrier): 11.24 -> 11.05 us at 640x640. In the register-kept kernel (its
// staging tiles as u23) it measured 0.5-2 % slower, so that kernel keeps
// the direct stores of waves 2-3's rows.
template <bool AFTER_STATE>
__device__ __forceinline__ void publish_summary(const FusedArgs& a, Smem& sm, const f4 (&S)[4],
                                                long long slot, int j, unsigned int ep, int w,
                                                int lane, float* u23 = nullptr)
{
    const int r = lane & 15, g = lane >> 4;
    const int tid = 64 * w + lane;
    // Every chunk load has landed (or reads past the end): retire them all
    // here, so that no later wait on a reused register waits for these stores.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    if (AFTER_STATE) lds_barrier();
    float* u01 = reinterpret_cast<float*>(AFTER_STATE ? sm.KtT : sm.ST0);
    if (w < 2 || u23) {
        float* dst = w < 2 ? u01 : u23;
        const int rw = 16 * (w & 1);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[(rw + 4 * g + e) * kU01 + 16 * jt + r] = S[jt][e];
    }
    if (tid < kMaxSpans) sm.tags[tid] = (ep + 1u) & 0xFFu;
    // wave 0 has waited for its loads, the staged header among them
    if (w == 0 && lane == 0 && !ws_header_ok(a, sm.hdr)) sm.wsbad = 1;
    lds_barrier();
    // an untrusted workspace: nothing is published (the caller takes the
    // failure path); the fault hook silences span 0 of every sequence
    if (w >= 2 && !sm.wsbad && !(a.fault && j == 0)) {
        const unsigned int tag = sm.tags[j];
        const int ns = a.n_spans, lo = a.slice_log2;
        const int ow = owner_region_words(ns, lo);
        const long long seq_base = (slot - j) / ns * agg_seq_words(ns);
        const __amdgpu_buffer_rsrc_t rs = rsrc(a.agg + seq_base, (int)(agg_seq_words(ns) * 4));
        // word of state element (row i, column col) in the owner-major layout:
        // owner i >> lr (2^lr rows each), then span j's slice, row and column
        const int lr = lo - 6;
        auto row_word = [&](int i) {
            return (i >> lr) * ow + (j << lo) + ((i & ((1 << lr) - 1)) << 6);
        };
        if (!u23) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int base = 4 * (row_word(16 * w + 4 * g + e) + r);
#pragma unroll
                for (int jt = 0; jt < 4; ++jt) st_dev1(rs, base + 64 * jt, ll_word(S[jt][e], tag));
            }
        }
        // rows from LDS (0-31, and 32-63 with u23), 16 B per lane: row q >> 4,
        // columns 4 (q & 15) .. +3
        const int nk = u23 ? 8 : 4;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k >= nk) continue;
            const int q = tid - 128 + 128 * k;
            const int row = q >> 4, c4 = 4 * (q & 15);
            // k < 4: rows 0-31 (u01); k >= 4: rows 32-63 (u23)
            const f4 x = *reinterpret_cast<const f4*>((k < 4 ? u01 : u23) + (row & 31) * kU01 + c4);
            u4 t;
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = ll_word(x[e], tag);
            st_dev4(rs, 4 * (row_word(row) + c4), t);
        }
        if (w == 2) {
            // decay of state row `lane`: owner (64 lane) >> lo, row within its slice
            const int o = (kD * lane) >> lo, ri = lane - (o << (lo - 6));
            st_dev1(rs, 4 * (o * ow + (ns << lo) + (j << (lo - 6)) + ri),
                    ll_word(ex2(sm.Pend[lane]), tag));
        }
    }
}

// Intra-chunk outputs kept through the exchange: fp32 for spans of up to two
// chunks, packed fp16 beyond (the register budget of long spans); the rounding
// is below the output's own fp16 rounding.
template <int SPAN>
struct KeptOut {
    static constexpr bool kHalf = SPAN > 2;
    f4 f[kHalf ? 1 : 4];
    h4 hv[kHalf ? 4 : 1];
    __device__ __forceinline__ void put(const f4 (&O)[4])
    {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (kHalf) hv[jt] = pack4(O[jt], 1.f);
            else f[jt] = O[jt];
        }
    }
    __device__ __forceinline__ void get(f4 (&O)[4]) const
    {
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
            if (kHalf) {
#pragma unroll
                for (int e = 0; e < 4; ++e) O[jt][e] = (float)hv[jt][e];
            } else {
                O[jt] = f[jt];
            }
        }
    }
};

// Local pass of a one-chunk span: intra-chunk outputs into K and the
// correction operand Qs = q 2^b for the incoming state; final local state in S;
// the summary is published right after the state update.
template <int SPAN>
__device__ __forceinline__ void keep_pass1(const FusedArgs& a, Smem& sm, const ChunkRegs& R, int b,
                                           int h, int c_first, int w, int lane, f4 (&S)[4],
                                           KeptOut<SPAN> (&K)[SPAN], h8 (&Qs)[SPAN][2],
                                           long long slot, int j, unsigned int ep)
{
    const int g = lane >> 4;
    ChunkTmp T;
    h8 Qt[2];
    chunk_front<true>(a, sm, R, w, lane, 0, S, false, Qt, T);
    publish_summary<true>(a, sm, S, slot, j, ep, w, lane, reinterpret_cast<float*>(sm.ST0));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
        Qs[0][hh] = Qt[hh] * *reinterpret_cast<const h8*>(&sm.cp16[32 * hh + 8 * g]);
    f4 O[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) O[n] = f4{0.f, 0.f, 0.f, 0.f};
    chunk_back(sm, a, b, h, c_first * kC, w, lane, false, O, Qt, T);
    K[0].put(O);
}

// Local pass of a span of NC >= 2 chunks, as a loop (one copy of the chunk
// code, for the instruction cache). One register set: chunk c + 1 is loaded
// as soon as chunk c's front half has consumed its registers. The intra-chunk
// outputs (fp16) and Qs = q 2^{b + P_c} (P_c: log2 decay from the span start
// to chunk c) of every chunk are parked in this workgroup's slots of the
// workspace, 64 bytes per thread per chunk; the summary is published right
// after the last state update.
__device__ __forceinline__ u4* park_slot(const FusedArgs& a, int c)
{
    return a.park + ((size_t)blockIdx.x * kMaxKeep + c) * (kThreads * 4) + 4 * threadIdx.x;
}

template <int NC>
__device__ __forceinline__ void keep_pass_loop(const FusedArgs& a, Smem& sm, ChunkRegs& R, int b,
                                               int h, int c_first, int w, int lane, f4 (&S)[4],
                                               long long slot, int j, unsigned int ep)
{
    for (int c = 0; c < NC; ++c) {
        // per-lane addresses are recomputed inside the loop instead of being
        // hoisted and held in registers across it
        asm volatile("" : "+v"(lane));
        const int g = lane >> 4;
        ChunkTmp T;
        h8 Qt[2];
        chunk_front<true>(a, sm, R, w, lane, c, S, c > 0, Qt, T);
        // never under a branch; past the span's end reads zeros
        load_chunk<true>(a, b, h, c + 1 < NC ? (c_first + c + 1) * kC : a.L, w, lane, R);
        if (c + 1 == NC) publish_summary<true>(a, sm, S, slot, j, ep, w, lane);
        h8 qs[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            qs[hh] = Qt[hh] * *reinterpret_cast<const h8*>(&sm.cp16[32 * hh + 8 * g]);
        f4 O[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) O[n] = f4{0.f, 0.f, 0.f, 0.f};
        chunk_back(sm, a, b, h, (c_first + c) * kC, w, lane, c > 0, O, Qt, T);
        u4* pk = park_slot(a, c);
        pk[0] = __builtin_bit_cast(u4, h8{(_Float16)O[0][0], (_Float16)O[0][1], (_Float16)O[0][2],
                                          (_Float16)O[0][3], (_Float16)O[1][0], (_Float16)O[1][1],
                                          (_Float16)O[1][2], (_Float16)O[1][3]});
        pk[1] = __builtin_bit_cast(u4, h8{(_Float16)O[2][0], (_Float16)O[2][1], (_Float16)O[2][2],
                                          (_Float16)O[2][3], (_Float16)O[3][0], (_Float16)O[3][1],
                                          (_Float16)O[3][2], (_Float16)O[3][3]});
        pk[2] = __builtin_bit_cast(u4, qs[0]);
        pk[3] = __builtin_bit_cast(u4, qs[1]);
    }
}

// Boundary exchange of one span (workgroup j of sequence local_seq): owners
// fold their slice of every span's summary and write each span's incoming
// state; every workgroup then reads its own incoming state and advances its
// slot's epoch. The state is returned in Sin (C layout: rows 16w + 4g + e,
// columns 16jt + r) and, when stage_st0, also staged in ST0 (fp16,
// transposed). Every wave must have finished with the chunk tiles' contents:
// they become scratch.
// final_state of sequence seq: dk x 64 fp32; rows past dk (the zero padding
// of a 32-wide key dim) fall outside the resource, and a null final_state
// gives an empty one (stores dropped)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t final_rsrc(const FusedArgs& a, int seq)
{
    return rsrc(a.final_state + (a.final_state ? (long long)seq * a.dk * kD : 0),
                a.final_state ? a.dk * kD * 4 : 0);
}

// ---- workspace header (gla_ws.h) and the failure paths ------------------------
// After a successful exchange, workgroup 0 records the layout in a workspace
// that was still clean. Every workgroup of the launch has read the header by
// then, or reads either value, which both admit this layout.
__device__ __forceinline__ void mark_ws_header(const FusedArgs& a, const unsigned int* hv, int tid)
{
    if (blockIdx.x == 0 && tid == 0 && hv[kWsMagicWord] == kWsClean) {
        const __amdgpu_buffer_rsrc_t rh = rsrc(a.hdr, kWsHeaderBytes);
        __builtin_amdgcn_raw_buffer_store_b32(a.layout, rh, 4 * kWsLayoutWord, 0, kDevScope);
        __builtin_amdgcn_raw_buffer_store_b32(~a.layout, rh, 4 * kWsLayoutCheck, 0, kDevScope);
        __builtin_amdgcn_raw_buffer_store_b32(kWsFused, rh, 4 * kWsMagicWord, 0, kDevScope);
    }
}
// A launch on an untrusted workspace publishes nothing and waits for nothing:
// it flags the header and writes NaN to every output row of its span and (span
// 0) to the sequence's final state.
__device__ void fail_untrusted(const FusedArgs& a, int b, int h, int seq, int j, int c_first,
                               int n_c, int w, int lane)
{
    const int tid = 64 * w + lane;
    if (tid == 0) atomicOr(a.hdr + kWsErrWord, kWsErrState);
    const u4 nan4 = {0x7E007E00u, 0x7E007E00u, 0x7E007E00u, 0x7E007E00u};
    for (int c = 0; c < n_c; ++c) {
        const long long off = row_offset(a, b, h, (c_first + c) * kC + 16 * w + (lane & 15));
        if (off >= 0) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *reinterpret_cast<u4*>(a.out + off + 8 * (lane >> 4) + 32 * hh) = nan4;
        }
    }
    if (j == 0) {
        const __amdgpu_buffer_rsrc_t rf = final_rsrc(a, seq);
        for (int e = tid; e < kD * kD; e += kThreads)
            __builtin_amdgcn_raw_buffer_store_b32(0x7FC00000u, rf, 4 * e, 0, 0);
    }
}

// Every wait of the exchange is bounded by a deadline on the chip's 100 MHz
// real-time counter (a.wait_ticks per poll loop). A wait that passes it gives
// up: the error word of the workspace header records it, an owner hands NaN
// incoming states (with the expected tags, so that its readers stop waiting)
// and a NaN final state to its slice, and a reader that gives up, or receives
// NaN, makes its workgroup write NaN outputs. Returns that poison flag.
__device__ __forceinline__ unsigned long long now_ticks() { return __builtin_amdgcn_s_memrealtime(); }

__device__ __forceinline__ bool exchange(const FusedArgs& a, Smem& sm, int local_seq, int seq, int j,
                                         long long seq_slot, int w, int lane, f4 (&Sin)[4],
                                         bool stage_st0)
{
    const int tid = 64 * w + lane;
    const int r = lane & 15, g = lane >> 4;
    if (tid == 0) sm.poison = 0;
    lds_barrier();   // every wave is done with the chunk tiles
    // The chunk tiles are free now: 45 KB of LDS scratch for the exchange.
    unsigned char* scr = reinterpret_cast<unsigned char*>(sm.Kh);
    const int ns = a.n_spans;
    const int lo = a.slice_log2;   // 2^lo state elements per owner
    if (j < (kD * kD >> lo)) {
        const int e_first = j << lo;
        const int lrows = lo - 6;                      // log2 of state rows in the slice
        const int ow = owner_region_words(ns, lo);
        const unsigned int* src = a.agg + local_seq * agg_seq_words(ns) + (long long)j * ow;
        unsigned int* ubuf = reinterpret_cast<unsigned int*>(scr);   // [ns][2^lo] U, [ns][rows] D
        unsigned int* s0buf = ubuf + ow;                              // initial state of the slice
        const int lq = lo - 2;                         // log2 of 16 B pieces per span
        const int nl = ow >> 2;
        // Fold, one state element per thread: the slice's E = 2^lo elements,
        // with P = 256 / E contiguous span ranges per element (combined through
        // LDS) when E < 256, else E / 256 elements per thread in turn. Words are
        // checked for their tag as the fold reads them; any stale word sends
        // the owner back to poll. Every span's incoming state and the final
        // state go from the fold straight to their global slots.
        const int lT = lo < 8 ? 8 - lo : 0;            // log2 P
        const int P = 1 << lT;
        const int per = (ns + P - 1) >> lT;            // spans per range
        const int lW = lo < 8 ? lo : 8;                // log2 elements per pass
        const int ei = tid & ((1 << lW) - 1), p = tid >> lW;
        const int m_lo = min(p * per, ns), m_hi = min(m_lo + per, ns);
        const int n_pass = 1 << (lo - lW);
        float* compA = reinterpret_cast<float*>(scr + kScanD + 2048);   // [256]
        float* compB = reinterpret_cast<float*>(scr + kScanD + 3072);   // [256]
        // the initial state's slice, staged with the first poll
        const float* s0 = reinterpret_cast<const float*>(s0buf);
        const __amdgpu_buffer_rsrc_t rs =
            rsrc(reinterpret_cast<const unsigned char*>(a.sin) + seq_slot * kSinSlotBytes, ns * kSinSlotBytes);
        const __amdgpu_buffer_rsrc_t rf = final_rsrc(a, seq);
        // the decays of every (span, row) of the slice, tag-checked and decoded
        // once into LDS floats (dfl), so that the fold reads plain values
        // (everything the fold uses lies below ST0, the last chunk tile, so
        // that the incoming state can be staged there while other waves of
        // the workgroup still fold: the region ends by 33.3 KB, dfl at
        // 33.5 KB, compA and compB up to 36 KB)
        float* dfl = reinterpret_cast<float*>(scr + kScanD + 1536);   // [ns << lrows] <= 128
        const int nd = ns << lrows;
        // When every span slot of the sequence expects the same tag (the
        // steady state: the slots' epochs advance together), the folds take
        // it from a register instead of reading the tag table per span.
        const unsigned int tag0 = sm.tags[0];
        const bool uni = __all(lane >= ns || sm.tags[lane] == tag0);
        // fold spans [m0, m1) of element e from `run`, checking the tags
        auto fold = [&](int e, int m0, int m1, float& A, float& run, bool& ok, auto uniform) {
            constexpr bool UNI = decltype(uniform)::value;
            const int su = 1 << lo, sd = 1 << lrows;
            const unsigned int* pu = ubuf + (m0 << lo) + e;
            const float* pd = dfl + (m0 << lrows) + (e >> 6);
            const unsigned int* pt = sm.tags + m0;
            int m = m0;
            for (; m + 4 <= m1; m += 4) {
                unsigned int xu[4], tg[4];
                float d[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    xu[k] = pu[k * su];
                    d[k] = pd[k * sd];
                    tg[k] = UNI ? tag0 : pt[k];
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    ok &= ll_ok(xu[k], tg[k]);
                    A *= d[k];
                    run = d[k] * run + ll_value(xu[k]);
                }
                pu += 4 * su;
                pd += 4 * sd;
                pt += 4;
            }
            for (; m < m1; ++m) {
                const unsigned int xu = *pu, tg = UNI ? tag0 : *pt;
                const float d = *pd;
                ok &= ll_ok(xu, tg);
                A *= d;
                run = d * run + ll_value(xu);
                pu += su;
                pd += sd;
                ++pt;
            }
        };
        float run0 = 0.f;   // ranged fold: the initial state of my element
        const unsigned long long t_start = now_ticks();
        bool gave_up = false;
        for (unsigned int polls = 0;; ++polls) {
            {   // every wave loads a share of the region
                for (int k0 = 64 * w; k0 < nl; k0 += 256) {
                    if (k0 + lane < nl)
                        __builtin_amdgcn_global_load_lds(src + 4 * (k0 + lane), ubuf + 4 * k0, 16, 0,
                                                         kDevScope);
                }
                if (a.init && polls == 0) {
                    // dk x 64 per sequence; the padded rows read zeros
                    const __amdgpu_buffer_rsrc_t ri =
                        rsrc(a.init + (long long)seq * a.dk * kD, a.dk * kD * 4);
                    for (int k0 = 64 * w; k0 < (1 << lq); k0 += 256) {
                        if (k0 + lane < (1 << lq))
                            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                                ri, (__attribute__((address_space(3))) void*)(s0buf + 4 * k0), 16,
                                4 * (e_first + 4 * (k0 + lane)), 0, 0, 0);
                    }
                }
                __builtin_amdgcn_s_waitcnt(0x0F70);
            }
            if (tid == 0) {
                sm.stale = 0;
                sm.dstale = 0;
            }
            bool ok = true;
            lds_barrier();
            if (tid < nd) {
                const unsigned int x = ubuf[(ns << lo) + tid];
                if (!ll_ok(x, sm.tags[tid >> lrows])) {
                    ok = false;
                    sm.dstale = 1;
                }
                dfl[tid] = ll_value(x);
            }
            lds_barrier();
            if (P == 1) {
                // the whole fold in one pass, from the initial state. The
                // incoming state of span m depends on the decays and on U of
                // spans 0 .. m-1 only: it is stored once those words have
                // passed their checks, so a stale pass stores only correct
                // words (a later pass stores them again, unchanged)
                const bool d_ok = sm.dstale == 0;
                auto fold1 = [&](auto uniform) {
                  for (int ps = 0; ps < n_pass; ++ps) {
                    const int e = (ps << 8) + tid;
                    float run = a.init ? s0[e] : 0.f;
                    bool mine = d_ok;
                    const unsigned int* pu = ubuf + e;
                    const float* pd = dfl + (e >> 6);
                    int voff = 2 * (e_first + e);
#pragma unroll 4
                    for (int m = 0; m < ns; ++m) {
                        const unsigned int xu = *pu, tg = decltype(uniform)::value ? tag0 : sm.tags[m];
                        const float d = *pd;
                        if (mine)
                            __builtin_amdgcn_raw_buffer_store_b16(sin_word(run, tg), rs, voff, 0, kDevScope);
                        mine = mine && ll_ok(xu, tg);
                        run = d * run + ll_value(xu);
                        pu += 1 << lo;
                        pd += 1 << lrows;
                        voff += kSinSlotBytes;
                    }
                    if (mine)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(run), rf,
                                                              4 * (e_first + e), 0, 0);
                    ok = ok && mine;
                  }
                };
                if (uni)
                    fold1(std::true_type{});
                else
                    fold1(std::false_type{});
            } else {
                // my range's product of decays and fold from zero
                float A = 1.f, run = 0.f;
                if (uni)
                    fold(ei, m_lo, m_hi, A, run, ok, std::true_type{});
                else
                    fold(ei, m_lo, m_hi, A, run, ok, std::false_type{});
                compA[tid] = A;
                compB[tid] = run;
                run0 = a.init ? s0[ei] : 0.f;
            }
            if (!__all(ok) && lane == 0) sm.stale = 1;
            if (tid == 0) sm.expired = (now_ticks() - t_start) > a.wait_ticks ? 1 : 0;
            lds_barrier();
            const bool stale = sm.stale;
            if (!stale) break;
            if (sm.expired) {   // (read by every thread before tid 0 rewrites it)
                gave_up = true;
                break;
            }
            lds_barrier();   // every thread has read the flags before they are reset
            __builtin_amdgcn_s_sleep(2);
        }
        if (gave_up) {
            // NaN incoming states for every span of the slice, with the tags
            // their readers expect, and a NaN final state
            if (tid == 0) atomicOr(a.hdr + kWsErrWord, kWsErrExchange);
            const unsigned short nanw = 0x7E00u;
            for (int e = tid; e < (1 << lo); e += kThreads) {
                int voff = 2 * (e_first + e);
                for (int m = 0; m < ns; ++m, voff += kSinSlotBytes)
                    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(nanw | (sm.tags[m] & 1u)),
                                                          rs, voff, 0, kDevScope);
                __builtin_amdgcn_raw_buffer_store_b32(0x7FC00000u, rf, 4 * (e_first + e), 0, 0);
            }
        } else if (P > 1) {
            // the ranges before mine (at most three), from the initial state;
            // then my range again, writing the incoming states
            float run = run0;
#pragma unroll
            for (int pp = 0; pp < 3; ++pp) {
                if (pp < p) {
                    const float ca = compA[(pp << lW) + ei], cb = compB[(pp << lW) + ei];
                    run = ca * run + cb;
                }
            }
            // every word has passed its tag check: each span's incoming
            // state goes straight from the fold to its slot, and the last
            // range ends with the final state
            auto pass2 = [&](auto uniform) {
                const unsigned int* pu = ubuf + (m_lo << lo) + ei;
                const float* pd = dfl + (m_lo << lrows) + (ei >> 6);
                int voff = m_lo * kSinSlotBytes + 2 * (e_first + ei);
#pragma unroll 4
                for (int m = m_lo; m < m_hi; ++m) {
                    const unsigned int xu = *pu;
                    const float d = *pd;
                    const unsigned int tg = decltype(uniform)::value ? tag0 : sm.tags[m];
                    __builtin_amdgcn_raw_buffer_store_b16(sin_word(run, tg), rs, voff, 0, kDevScope);
                    run = d * run + ll_value(xu);
                    pu += 1 << lo;
                    pd += 1 << lrows;
                    voff += kSinSlotBytes;
                }
            };
            if (uni)
                pass2(std::true_type{});
            else
                pass2(std::false_type{});
            if (p == P - 1)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(run), rf, 4 * (e_first + ei), 0, 0);
        }
    }

    // my incoming state S_in: each wave polls its own rows straight into
    // registers until every word carries the slot's tag; span 0 reads zeros
    // like the others so that its epoch, too, advances only once every owner
    // has read it
    {
        const unsigned int tag = sm.tags[j];
        const __amdgpu_buffer_rsrc_t rsn =
            rsrc(reinterpret_cast<const unsigned char*>(a.sin) + (seq_slot + j) * kSinSlotBytes, kSinSlotBytes);
        const unsigned long long t_start = now_ticks();
        bool bad = false;
        for (;;) {
            asm volatile("" ::: "memory");   // a fresh load every round
            unsigned short x[4][4];
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x[jt][e] = __builtin_amdgcn_raw_buffer_load_b16(
                        rsn, 2 * ((16 * w + 4 * g + e) * kD + 16 * jt + r), 0, kDevScope);
            bool ok = true;
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ok &= sin_ok(x[jt][e], tag);
                    Sin[jt][e] = sin_value(x[jt][e]);
                }
            if (__all(ok)) break;
            if (now_ticks() - t_start > a.wait_ticks) {   // wave-uniform
                if (lane == 0) atomicOr(a.hdr + kWsErrWord, kWsErrExchange);
                bad = true;
                break;
            }
            __builtin_amdgcn_s_sleep(kPollSleep);
        }
        // a NaN incoming state (an owner that gave up) poisons the workgroup too
#pragma unroll
        for (int jt = 0; jt < 4; ++jt)
#pragma unroll
            for (int e = 0; e < 4; ++e) bad |= __builtin_isnan(Sin[jt][e]);
        if (__any(bad) && lane == 0) sm.poison = 1;
        // ST0 is outside the fold's scratch: stage right away
        if (stage_st0) {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt) st4(sm.ST0, 16 * jt + r, 16 * w + 4 * g, pack4(Sin[jt], 1.f));
        }
        // Every owner has read this slot's epoch (it wrote S_in after reading
        // the epochs), and so has every wave here: advance it. The barrier
        // also makes the staged state (and anything the caller wrote to LDS
        // before the exchange) visible, and frees the chunk tiles.
        lds_barrier();
        if (tid == 0) __hip_atomic_store(a.epoch + seq_slot + j, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return sm.poison != 0;
}

// ---------------------------------------------------------------------------
// VAR: which optional parts the kernel has code for: kPlain none, kExtras the
// initial state and the output gate, kLowRank those and the low-rank gate.
// The kernel's copy of the arguments has constant nulls for the parts it
// lacks, which removes their branches (and code) from the lighter variants.
constexpr int kPlain = 0, kExtras = 1, kLowRank = 2;
template <int VAR>
__device__ __forceinline__ FusedArgs variant_args(const FusedArgs& in)
{
    {
        // one word of each 64-byte line of the arguments, in one batch: every
        // later argument load hits the scalar cache
        const unsigned int* aw = reinterpret_cast<const unsigned int*>(&in);
        asm volatile("" ::"s"(aw[0]), "s"(aw[16]), "s"(aw[32]), "s"(aw[48]));
    }
    FusedArgs a = in;
    if (VAR < kLowRank) a.z = nullptr;
    if (VAR < kExtras) {
        a.init = nullptr;
        a.gate = nullptr;
    }
    return a;
}

template <int SPAN, bool KEEP, int VAR>
__global__ void __launch_bounds__(kThreads, 3)
gla_fused_kernel(FusedArgs a_arg)
{
    const FusedArgs a = variant_args<VAR>(a_arg);
    static_assert(!KEEP || SPAN <= kMaxKeep, "a kept span holds at most kMaxKeep chunks");
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;

    const int local_seq = blockIdx.x / a.n_spans;
    const int j = blockIdx.x - local_seq * a.n_spans;
    const int seq = a.seq0 + local_seq;
    const int b = seq / a.H, h = seq - (seq / a.H) * a.H;
    const int span = KEEP ? SPAN : a.span;
    const int c_first = j * span;
    const int n_c = min(span, a.n_chunks - c_first);
    __builtin_assume(n_c >= 1);   // every span starts inside the sequence

    // Epochs of the sequence's span slots (thread t < n_spans reads slot t;
    // the rest read zeros past the end), then the first chunk. The epochs are
    // first used at the publish, so nothing waits for them before.
    const long long seq_slot = (long long)local_seq * a.n_spans;
    const unsigned int ep = __builtin_amdgcn_raw_buffer_load_b32(
        rsrc(a.epoch + seq_slot, 4 * a.n_spans), 4 * tid, 0, kDevScope);
    stage_ws_header(a, sm.hdr, w, lane);   // checked at the publish
    // RMSNorm weight of the output epilogue (an empty resource without a gate)
    const float nwr = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rsrc(a.norm_w, a.gate ? 4 * kD : 0), 4 * (tid & (kD - 1)), 0, 0));
    ChunkRegs cur;
    load_chunk<KEEP>(a, b, h, c_first * kC, w, lane, cur);
    if (tid == 0) sm.wsbad = 0;   // ordered by the local pass's first barrier
    if (tid < kD) {
        sm.P[0][tid] = 0.f;
        sm.Pend[tid] = 0.f;
    }
    if (a.z) {
        fill_gate_tables(a, h, tid);
        lds_barrier();
    }

    // ---- 1. local pass --------------------------------------------------------
    // The span summary is published right after the last chunk's state update,
    // before that chunk's outputs, so the exchange overlaps them.
    f4 S[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) S[n] = f4{0.f, 0.f, 0.f, 0.f};
    // kept intra-chunk output and correction operand of a one-chunk span
    KeptOut<1> K[1];
    h8 Qs[1][2];
    if (KEEP) {
        // No branch on the chunk count: a span that ends early runs empty
        // chunks (zero rows leave the state and the decay unchanged and their
        // outputs are never stored), so every workgroup does the same work and
        // no path past the publish stores has a chunk load in flight (a wait
        // for one would also wait for the stores).
        if constexpr (SPAN == 1)
            keep_pass1<1>(a, sm, cur, b, h, c_first, w, lane, S, K, Qs, seq_slot + j, j, ep);
        else
            keep_pass_loop<(KEEP ? SPAN : 1)>(a, sm, cur, b, h, c_first, w, lane, S, seq_slot + j,
                                              j, ep);
    } else {
        h8 qdummy[2];
        ChunkTmp T;
        for (int c = 0; c < n_c; ++c) {
            int ln = lane;
            asm volatile("" : "+v"(ln));   // addresses recomputed per chunk, not held live
            chunk_front<false>(a, sm, cur, w, ln, c, S, false, qdummy, T);
            load_chunk<false>(a, b, h, c + 1 < n_c ? (c_first + c + 1) * kC : a.L, w, lane, cur);
        }
        publish_summary<false>(a, sm, S, seq_slot + j, j, ep, w, lane);
    }
    if (sm.wsbad) {   // set before the publish's barrier
        fail_untrusted(a, b, h, seq, j, c_first, n_c, w, lane);
        return;
    }

    // ---- 2. boundary scan across the sequence's spans -------------------------
    // The first `owners` workgroups (a power of two <= n_spans) each own a
    // slice of 2^slice_log2 state elements: they read that slice of every
    // span's U and D, fold S_in[m+1] = D_m S_in[m] + U_m through the spans, and
    // write every span's incoming state (and the final state) for the slice.
    // Then every workgroup reads its own S_in.
    u4 zg[2];   // the one-chunk span's gate, fetched while the exchange runs
    if (KEEP && SPAN == 1) load_gate(a, b, h, c_first * kC, w, lane, zg);
    // the incoming state is nonzero past the first span, or with an initial state
    const bool has_in = j > 0 || a.init != nullptr;
    if (tid < kD) sm.nw[tid] = nwr;   // the exchange's last barrier orders it
    f4 Sin[4];
    const bool poison = exchange(a, sm, local_seq, seq, j, seq_slot, w, lane, Sin, KEEP && has_in);
    if (!poison) mark_ws_header(a, sm.hdr, tid);

    // ---- 3. outputs -----------------------------------------------------------
    if (KEEP) {
        if constexpr (SPAN == 1) {
            f4 O[4];
            K[0].get(O);
            if (has_in) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt)
                        O[jt] = mfma(ld8(sm.ST0, 16 * jt + r, 32 * hh + 8 * g), Qs[0][hh], O[jt]);
            }
            store_out(sm, a, b, h, c_first * kC, w, lane, O, zg, poison);
        } else {
            // parked chunks: the next chunk's slot loads while this one finishes
            u4 pk[4], pn[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) pk[k] = park_slot(a, 0)[k];
            for (int c = 0; c < n_c; ++c) {
                f4 O[4];
                h8 qs[2];
#pragma unroll
                for (int k = 0; k < 4; ++k) pn[k] = park_slot(a, c + 1 < SPAN ? c + 1 : c)[k];
                const h8 o01 = __builtin_bit_cast(h8, pk[0]), o23 = __builtin_bit_cast(h8, pk[1]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    O[0][e] = (float)o01[e];
                    O[1][e] = (float)o01[4 + e];
                    O[2][e] = (float)o23[e];
                    O[3][e] = (float)o23[4 + e];
                }
                qs[0] = __builtin_bit_cast(h8, pk[2]);
                qs[1] = __builtin_bit_cast(h8, pk[3]);
                u4 z[2];
                if (a.gate) load_gate(a, b, h, (c_first + c) * kC, w, lane, z);
                if (has_in) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int jt = 0; jt < 4; ++jt)
                            O[jt] = mfma(ld8(sm.ST0, 16 * jt + r, 32 * hh + 8 * g), qs[hh], O[jt]);
                }
                store_out(sm, a, b, h, (c_first + c) * kC, w, lane, O, z, poison);
#pragma unroll
                for (int k = 0; k < 4; ++k) pk[k] = pn[k];
            }
        }
    } else {
        // stream the span again from its incoming state
#pragma unroll
        for (int n = 0; n < 4; ++n) S[n] = Sin[n];
        lds_barrier();   // the norm weight is in LDS
        if (has_in) {
#pragma unroll
            for (int jt = 0; jt < 4; ++jt)
                st4(sm.ST0, 16 * jt + r, 16 * w + 4 * g, pack4(S[jt], 1.f));
        }
        load_chunk<true>(a, b, h, c_first * kC, w, lane, cur);
        for (int c = 0; c < n_c; ++c) {
            int ln = lane;
            asm volatile("" : "+v"(ln));   // addresses recomputed per chunk, not held live
            f4 Oc[4];
            h8 qt[2];
#pragma unroll
            for (int n = 0; n < 4; ++n) Oc[n] = f4{0.f, 0.f, 0.f, 0.f};
            ChunkTmp T;
            u4 z[2];
            if (a.gate) load_gate(a, b, h, (c_first + c) * kC, w, ln, z);
            chunk_front<true>(a, sm, cur, w, ln, kMaxKeep, S, c > 0, qt, T);
            load_chunk<true>(a, b, h, c + 1 < n_c ? (c_first + c + 1) * kC : a.L, w, ln, cur);
            chunk_back(sm, a, b, h, (c_first + c) * kC, w, ln, has_in || (c > 0), Oc, qt, T);
            store_out(sm, a, b, h, (c_first + c) * kC, w, ln, Oc, z, poison);
        }
    }
}

// ---------------------------------------------------------------------------
// Register-kept spans: every chunk's intra-chunk outputs (fp16) and correction
// operand Qs stay in registers through the exchange (two workgroups per CU),
// and the next chunk's g, k and v are staged in LDS by DMA while the current
// chunk computes, so that a chunk's loads are in flight for a whole chunk.
struct SmemRK {
    Smem s;
    // g, k, v of one chunk, 64 rows of eight 16-byte blocks; block m of row t
    // sits in slot m ^ (t & 7) (consecutive rows spread over the banks)
    _Float16 raw[3][kC * kD];
};

// Each wave stages its own 16 rows: lane l fetches row 16w + 8i + (l >> 3)
// (i = 0, 1), block (l & 7) ^ (row & 7), into slot l & 7. Rows past the
// sequence end read zeros.
__device__ __forceinline__ void dma_gkv(const FusedArgs& a, SmemRK& sk, int b, int h, int t0, int w,
                                        int lane)
{
    const __amdgpu_buffer_rsrc_t rg = batch_rsrc(a.lg, a, b, a.dk), rk = batch_rsrc(a.k, a, b, a.dk),
                                 rv = batch_rsrc(a.v, a, b);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row = 16 * w + 8 * i + (lane >> 3);
        const RowOff o = row_off(a, h, t0 + row, (lane & 7) ^ (row & 7));
        const int base = (16 * w + 8 * i) * kD;
        if (!a.z)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rg, (__attribute__((address_space(3))) void*)(sk.raw[0] + base), 16, o.key, 0, 0, kNT);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rk, (__attribute__((address_space(3))) void*)(sk.raw[1] + base), 16, o.key, 0, 0, kNT);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rv, (__attribute__((address_space(3))) void*)(sk.raw[2] + base), 16, o.val, 0, 0, kNT);
    }
}

// With the low-rank gate, raw[0] holds z instead of g: the wave's 16 rows of
// 16 floats, one DMA per wave (lane l: row 16w + (l >> 2), floats 4(l & 3) ..).
__device__ __forceinline__ void dma_z(const FusedArgs& a, SmemRK& sk, int b, int t0, int w, int lane)
{
    const int bytes = a.L * 64;
    const __amdgpu_buffer_rsrc_t rz = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.z + (long long)b * a.L * 16), (short)0, bytes, 0x00020000);
    const int t = t0 + 16 * w + (lane >> 2);
    const int voff = t < a.L ? scan_to_spatial(t, a.L, a.grid_h, a.grid_w, a.dir) * 64 + 16 * (lane & 3)
                             : bytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rz, (__attribute__((address_space(3))) void*)(sk.raw[0] + 16 * w * 32), 16, voff, 0, 0, kNT);
}

__device__ __forceinline__ u4 raw_ld(const _Float16* tile, int row, int blk)
{
    return *reinterpret_cast<const u4*>(tile + row * kD + 8 * (blk ^ (row & 7)));
}

// q of a chunk into registers, in the operand layout of load_chunk.
__device__ __forceinline__ void load_q(const FusedArgs& a, int b, int h, int t0, int w, int lane,
                                       u4 (&q)[2])
{
    const int t = t0 + 16 * w + (lane & 15);
    const __amdgpu_buffer_rsrc_t rq = batch_rsrc(a.q, a, b, a.dk);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) q[hh] = load16(rq, row_off(a, h, t, (lane >> 4) + 4 * hh).key);
}

template <int SPAN, int VAR>
__global__ void __launch_bounds__(kThreads, 2)
gla_fused_rk_kernel(FusedArgs a_arg)
{
    const FusedArgs a = variant_args<VAR>(a_arg);
    static_assert(SPAN >= 2 && SPAN <= kMaxKeep, "register-kept spans hold 2 .. kMaxKeep chunks");
    SmemRK& sk = *reinterpret_cast<SmemRK*>(smem_raw);
    Smem& sm = sk.s;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
    const int lane = tid & 63;
    const int r = lane & 15, g = lane >> 4;

    const int local_seq = blockIdx.x / a.n_spans;
    const int j = blockIdx.x - local_seq * a.n_spans;
    const int seq = a.seq0 + local_seq;
    const int b = seq / a.H, h = seq - (seq / a.H) * a.H;
    const int c_first = j * SPAN;
    const int n_c = min(SPAN, a.n_chunks - c_first);

    const long long seq_slot = (long long)local_seq * a.n_spans;
    const unsigned int ep = __builtin_amdgcn_raw_buffer_load_b32(
        rsrc(a.epoch + seq_slot, 4 * a.n_spans), 4 * tid, 0, kDevScope);
    const float nwr = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
        rsrc(a.norm_w, a.gate ? 4 * kD : 0), 4 * (tid & (kD - 1)), 0, 0));
    stage_ws_header(a, sm.hdr, w, lane);   // checked at the publish
    if (tid == 0) sm.wsbad = 0;            // ordered by the first chunk's barrier
    dma_gkv(a, sk, b, h, c_first * kC, w, lane);
    if (a.z) dma_z(a, sk, b, c_first * kC, w, lane);
    u4 qn[2];
    load_q(a, b, h, c_first * kC, w, lane, qn);
    if (tid < kD) {
        sm.P[0][tid] = 0.f;
        sm.Pend[tid] = 0.f;
    }
    if (a.z) fill_gate_tables(a, h, tid);   // the loop's first barrier orders it

    // ---- 1. local pass: SPAN chunks, always (past the sequence end the
    // staged rows are zeros: state and decay unchanged, outputs not stored)
    f4 S[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) S[n] = f4{0.f, 0.f, 0.f, 0.f};
    // kept per chunk: fp16 intra-chunk outputs (C layout) and Qs at index c.
    // The loop body is one copy of the chunk code; a scalar branch on c moves
    // the chunk's results into their slot (registers cannot be indexed, and
    // shifting the arrays instead costs 16 moves per kept chunk)
    h8 KO[SPAN][2], KQ[SPAN][2];
#pragma unroll 1
    for (int c = 0; c < SPAN; ++c) {
        int ln = lane;
        asm volatile("" : "+v"(ln));   // addresses recomputed per chunk, not held live
        const int rr = ln & 15, gg = ln >> 4;
        // this chunk's staged rows and q have landed; each wave reads only the
        // rows it staged itself, so only the first chunk needs a barrier (it
        // orders the set-up above, e.g. the gate tables)
        __builtin_amdgcn_s_waitcnt(0x0F70);
        if (c == 0) lds_barrier();
        ChunkRegs R;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            R.q[hh] = qn[hh];
            R.g[hh] = raw_ld(sk.raw[0], 16 * w + rr, 4 * hh + gg);
            R.k[hh] = raw_ld(sk.raw[1], 16 * w + rr, 4 * hh + gg);
            R.v[hh] = raw_ld(sk.raw[2], 16 * w + rr, 4 * hh + gg);
        }
        if (a.z) {   // z rows of the chunk: 16 floats per row, the lane's eight at 8 (gg & 1)
            const float* zr = reinterpret_cast<const float*>(sk.raw[0]) + (16 * w + rr) * 16 +
                              8 * (gg & 1);
            R.g[0] = *reinterpret_cast<const u4*>(zr);
            R.g[1] = *reinterpret_cast<const u4*>(zr + 4);
            R.valid = (c_first + c) * kC + 16 * w + rr < a.L;
        }
        h8 Qt[2];
        ChunkTmp T;
        // never under a branch; past the span's end reads zeros
        const int tn = c + 1 < SPAN ? (c_first + c + 1) * kC : a.L;
        chunk_front<true>(a, sm, R, w, ln, c, S, c > 0, Qt, T, [&]() {
            dma_gkv(a, sk, b, h, tn, w, ln);
            if (a.z) dma_z(a, sk, b, tn, w, ln);
            load_q(a, b, h, tn, w, ln, qn);
        });
        if (c + 1 == SPAN) publish_summary<true>(a, sm, S, seq_slot + j, j, ep, w, ln);
        h8 qs[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            qs[hh] = Qt[hh] * *reinterpret_cast<const h8*>(&sm.cp16[32 * hh + 8 * gg]);
        f4 O[4];
#pragma unroll
        for (int n = 0; n < 4; ++n) O[n] = f4{0.f, 0.f, 0.f, 0.f};
        chunk_back(sm, a, b, h, (c_first + c) * kC, w, ln, c > 0, O, Qt, T);
        const h8 o0 = h8{(_Float16)O[0][0], (_Float16)O[0][1], (_Float16)O[0][2], (_Float16)O[0][3],
                         (_Float16)O[1][0], (_Float16)O[1][1], (_Float16)O[1][2], (_Float16)O[1][3]};
        const h8 o1 = h8{(_Float16)O[2][0], (_Float16)O[2][1], (_Float16)O[2][2], (_Float16)O[2][3],
                         (_Float16)O[3][0], (_Float16)O[3][1], (_Float16)O[3][2], (_Float16)O[3][3]};
        // c is wave-uniform: one scalar branch picks the slot
#pragma unroll
        for (int i = 0; i < SPAN; ++i)
            if (i == c) {
                KO[i][0] = o0;
                KO[i][1] = o1;
                KQ[i][0] = qs[0];
                KQ[i][1] = qs[1];
            }
    }

    if (sm.wsbad) {   // set before the publish's barrier
        fail_untrusted(a, b, h, seq, j, c_first, n_c, w, lane);
        return;
    }

    // ---- 2. boundary exchange --------------------------------------------------
    const bool has_in = j > 0 || a.init != nullptr;
    f4 Sin[4];
    if (tid < kD) sm.nw[tid] = nwr;   // the exchange's last barrier orders it
    const bool poison = exchange(a, sm, local_seq, seq, j, seq_slot, w, lane, Sin, has_in);
    if (!poison) mark_ws_header(a, sm.hdr, tid);

    // ---- 3. outputs: O_c += Qs_c S_in (the state is in ST0) -----------------------
    // the gate of the next chunk loads while this one finishes
    u4 zc[2], zn[2];
    if (a.gate) load_gate(a, b, h, c_first * kC, w, lane, zc);
#pragma unroll
    for (int c = 0; c < SPAN; ++c) {
        if (a.gate && c + 1 < n_c) load_gate(a, b, h, (c_first + c + 1) * kC, w, lane, zn);
        if (c < n_c) {
            const int ki = c;
            f4 O[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                O[0][e] = (float)KO[ki][0][e];
                O[1][e] = (float)KO[ki][0][4 + e];
                O[2][e] = (float)KO[ki][1][e];
                O[3][e] = (float)KO[ki][1][4 + e];
            }
            if (has_in) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int jt = 0; jt < 4; ++jt)
                        O[jt] = mfma(ld8(sm.ST0, 16 * jt + r, 32 * hh + 8 * g), KQ[ki][hh], O[jt]);
            }
            store_out(sm, a, b, h, (c_first + c) * kC, w, lane, O, zc, poison);
        }
        zc[0] = zn[0];
        zc[1] = zn[1];
    }
}

// ---------------------------------------------------------------------------
// Zero fill, used instead of hipMemsetAsync so that it can sit in a captured graph.
__global__ void fill_zero_kernel(unsigned char* p, size_t n)
{
    const size_t n16 = n / 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        reinterpret_cast<u4*>(p)[i] = u4{0u, 0u, 0u, 0u};
    if (blockIdx.x == 0 && threadIdx.x < n - 16 * n16) p[16 * n16 + threadIdx.x] = 0;
}

// Workspace initialisation: zero everything past the header, then a clean
// header (error word 0, magic kWsClean).
__global__ void init_ws_kernel(unsigned char* p, size_t n)
{
    const size_t n16 = n / 16;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x + kWsHeaderBytes / 16; i < n16;
         i += (size_t)gridDim.x * blockDim.x)
        reinterpret_cast<u4*>(p)[i] = u4{0u, 0u, 0u, 0u};
    if (blockIdx.x == 0 && threadIdx.x < n - 16 * n16) p[16 * n16 + threadIdx.x] = 0;
    if (blockIdx.x == 0 && threadIdx.x < kWsHeaderBytes / 4)
        reinterpret_cast<unsigned int*>(p)[threadIdx.x] = threadIdx.x == kWsMagicWord ? kWsClean : 0u;
}

hipError_t init_workspace(void* p, size_t bytes, hipStream_t st)
{
    if (bytes < (size_t)kWsHeaderBytes) return hipErrorInvalidValue;
    if (((uintptr_t)p & 15) != 0) return hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    int blocks = (int)((n16 + 255) / 256);
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    unsigned char* base = (unsigned char*)p;
    void* args[] = {&base, &bytes};
    // the launch's own status (not an earlier, unrelated error of the thread)
    return hipLaunchKernel((const void*)init_ws_kernel, dim3(blocks), dim3(256), args, 0, st);
}

// Exchange wait limit and the give-up test hook (process-wide).
static std::atomic<unsigned int> g_wait_us{20000};
static std::atomic<int> g_fault{0};
void set_exchange_wait(unsigned int wait_us, int fault)
{
    g_wait_us.store(wait_us, std::memory_order_relaxed);
    g_fault.store(fault, std::memory_order_relaxed);
}
unsigned int exchange_wait_us() { return g_wait_us.load(std::memory_order_relaxed); }

// Ticks per microsecond of the counter the kernels read (s_memrealtime).
static unsigned long long wall_ticks_per_ms()
{
    static int cached = 0;
    if (cached == 0) {
        int dev = 0, khz = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
            khz < 1)
            khz = 100000;   // 100 MHz
        cached = khz;
    }
    return (unsigned long long)cached;
}

unsigned int fused_layout_word(const FusedPlan& p)
{
    // one exchange slot layout per (kernel family, state rows, spans per
    // sequence, sequences per launch)
    return 0x80000000u | ((unsigned int)(p.family & 3) << 28) | ((p.dk == 32 ? 1u : 0u) << 27) |
           ((unsigned int)p.seq_batch << 8) | (unsigned int)p.n_spans;
}

// Workgroups a plan may take as resident at once: 7/8 of the occupancy bound.
// The dispatcher spreads a launch's workgroups evenly over the shader engines
// rather than by their free slots, so a grid that needs every slot of the chip
// can leave workgroups waiting for others to finish; the exchange, which needs
// every workgroup of a launch running, would then time out.
long long resident_cap(int per_cu, int cus)
{
    return (long long)per_cu * cus * 7 / 8;
}

hipError_t fill_zero(void* p, size_t bytes, hipStream_t st)
{
    if (bytes == 0) return hipSuccess;
    if (((uintptr_t)p & 15) != 0) return hipErrorInvalidValue;
    const size_t n16 = bytes / 16;
    int blocks = (int)((n16 + 255) / 256);
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, (unsigned char*)p, bytes);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
bool fused_supported(const Shape& s)
{
    // d_v = 64; d_k = 64, or 32 (the pages' operator shape) zero-padded to 64
    // in the kernel; buffer offsets within one batch are 32-bit
    return (s.d_k == kD || s.d_k == 32) && s.d_v == kD && s.chunk == kC &&
           (long long)s.L * s.H * kD * 2 + 256 <= 0x7FFFFFFFLL;
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

// Kept spans (chunk registers, parking) are instantiated for these lengths;
// register-kept spans for 2 .. 7 (eight chunks' outputs overflow the registers).
static bool keep_span_ok(int span) { return span == 1 || span == 2 || span == 4 || span == 8; }
static bool rk_span_ok(int span) { return span >= 2 && span <= 7; }

template <int LR>
static const void* pick_variant(int span, bool keep, bool rk)
{
    if (rk) {
        switch (span) {
        case 2: return (const void*)gla_fused_rk_kernel<2, LR>;
        case 3: return (const void*)gla_fused_rk_kernel<3, LR>;
        case 4: return (const void*)gla_fused_rk_kernel<4, LR>;
        case 5: return (const void*)gla_fused_rk_kernel<5, LR>;
        case 6: return (const void*)gla_fused_rk_kernel<6, LR>;
        default: return (const void*)gla_fused_rk_kernel<7, LR>;
        }
    }
    if (!keep) return (const void*)gla_fused_kernel<1, false, LR>;
    switch (span) {
    case 1: return (const void*)gla_fused_kernel<1, true, LR>;
    case 2: return (const void*)gla_fused_kernel<2, true, LR>;
    case 4: return (const void*)gla_fused_kernel<4, true, LR>;
    default: return (const void*)gla_fused_kernel<8, true, LR>;
    }
}
static const void* pick_kernel(int span, bool keep, bool rk, int var)
{
    return var == kLowRank ? pick_variant<kLowRank>(span, keep, rk)
                           : var == kExtras ? pick_variant<kExtras>(span, keep, rk)
                                            : pick_variant<kPlain>(span, keep, rk);
}

// Dynamic LDS: the variant's Smem, then (low-rank gate) the gate tables.
static size_t gate_tab_offset(bool rk) { return ((rk ? sizeof(SmemRK) : sizeof(Smem)) + 15) / 16 * 16; }
static size_t smem_bytes(bool rk, int var)
{
    return var == kLowRank ? gate_tab_offset(rk) + sizeof(GateTab) : (rk ? sizeof(SmemRK) : sizeof(Smem));
}

// Workgroups of one variant that fit on a CU at once.
static int resident_per_cu(int span, bool keep, bool rk, int var)
{
    static int cache[3][3][kMaxKeep + 1] = {};
    int& c = cache[var][rk ? 2 : (keep ? 1 : 0)][(keep || rk) ? span : 0];
    if (c == 0) {
        const void* fn = pick_kernel(span, keep, rk, var);
        int n = 0;
        const size_t sh = smem_bytes(rk, var);
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
        if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, kThreads, sh);
        if (e != hipSuccess) {
            log_hip("occupancy query of a fused kernel", e);
            (void)hipGetLastError();   // do not leave it for a later call to report
            n = 1;
        }
        if (n < 1) n = 1;
        c = n;
    }
    return c;
}

// Test hook: GTR_GLA_MAX_RESIDENT=n caps the workgroups the plan takes as
// resident at once (so that a small shape needs several launches).
static long long resident_cap_from_env()
{
    if (const char* env = std::getenv("GTR_GLA_MAX_RESIDENT")) {
        const long long v = std::atoll(env);
        if (v > 0) return v;
    }
    return 0;
}

FusedPlan fused_plan(const Shape& s, int span_override, int rk_override, int var)
{
    FusedPlan p;
    p.var = var;
    const int n_seq = s.B * s.H;
    const int nc = s.n_chunks;
    const long long cap_env = resident_cap_from_env();
    auto capacity = [&](int span, bool keep, bool rk) {
        const long long cap = resident_cap(resident_per_cu(span, keep, rk, var), device_cus());
        return cap_env > 0 && cap_env < cap ? cap_env : cap;
    };
    auto fill = [&](int span, bool keep, bool rk = false) {
        p.span = span;
        p.keep = keep || rk;
        p.rk = rk;
        p.n_spans = (nc + span - 1) / span;
        const long long cap = capacity(span, keep, rk);
        // sequences per launch, so that every workgroup of a launch is resident
        long long per = cap / p.n_spans;
        if (per < 1) per = 1;
        p.seq_batch = (int)(per < n_seq ? per : n_seq);
        p.grid = p.seq_batch * p.n_spans;
        // owners: the largest power of two <= n_spans; each scans 4096 / owners elements
        int lg = 0;
        while ((2 << lg) <= p.n_spans) ++lg;
        p.slice_log2 = 12 - lg;
    };
    auto one_seq_fits = [&]() { return (long long)p.n_spans <= capacity(p.span, p.keep, p.rk); };
    if (span_override > 0) {
        if (rk_override > 0 && rk_span_ok(span_override)) {
            fill(span_override, false, true);
            if (one_seq_fits() && p.n_spans <= kMaxSpans) return p;
        }
        fill(span_override, keep_span_ok(span_override));
        while (!one_seq_fits() || p.n_spans > kMaxSpans) fill(p.span * 2, false);
        return p;
    }
    auto whole = [&]() { return p.seq_batch == n_seq && p.n_spans <= kMaxSpans; };
    // one chunk per workgroup when every chunk fits on the chip at once with
    // at most two workgroups per CU
    fill(1, true);
    const bool one_chunk_fits = whole();
    if (one_chunk_fits && p.grid <= 2 * device_cus()) return p;
    // else the shortest register-kept span whose whole grid is resident
    // (no outputs round-trip through memory); a third one-chunk workgroup per
    // CU (1024 x 1024 images: 768 workgroups) measured 3-4 % slower than
    // register-kept spans of two chunks; then parked spans
    for (int sp = 2; rk_span_ok(sp); ++sp) {
        fill(sp, false, true);
        if (whole()) return p;
    }
    if (one_chunk_fits) {
        fill(1, true);
        return p;
    }
    for (int sp = 2; sp <= kMaxKeep; sp *= 2) {
        fill(sp, true);
        if (whole()) return p;
    }
    // else streamed spans
    const long long cap = capacity(1, false, false);
    long long per_seq = cap / n_seq;
    if (per_seq < 1) per_seq = 1;
    if (per_seq > kMaxSpans) per_seq = kMaxSpans;
    fill((int)((nc + per_seq - 1) / per_seq), false);
    while (!one_seq_fits() || p.n_spans > kMaxSpans) fill(p.span * 2, false);
    return p;
}

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace: error word, then per exchange slot (sequence in launch, span): an
// epoch, the published summary and the incoming state; then, for kept spans of
// two or more chunks (keep_pass_loop), the parking slots (kMaxKeep chunks per
// workgroup).
static size_t park_bytes(const FusedPlan& p)
{
    return (p.keep && !p.rk && p.span >= 2) ? (size_t)p.grid * kMaxKeep * kThreads * sizeof(u4) * 4
                                            : 0;
}

size_t fused_workspace_bytes(const Shape& s, const FusedPlan& p)
{
    if (p.family == 2) return span_workspace_bytes(s, p);
    const size_t slots = (size_t)p.seq_batch * p.n_spans;
    return 256 + align256(slots * sizeof(unsigned int)) +
           align256((size_t)p.seq_batch * agg_seq_words(p.n_spans) * sizeof(unsigned int) +
                    slots * kSinSlotBytes) +
           park_bytes(p);
}

hipError_t launch_fused(const void* q, const void* k, const void* v, const void* lg,
                        const Shape& s, const Extras& x, const FusedPlan& p, void* out,
                        float* final_state, void* ws, hipStream_t st)
{
    if (p.family == 2)
        return launch_span(q, k, v, lg, s, x, p, out, final_state, ws, st, fused_layout_word(p),
                           g_fault.load(std::memory_order_relaxed),
                           (unsigned long long)g_wait_us.load(std::memory_order_relaxed) *
                               wall_ticks_per_ms() / 1000ull);
    FusedArgs a;
    a.init = x.init;
    a.gate = (const __half*)x.gate;
    a.norm_w = x.norm_w;
    a.eps = x.eps;
    a.z = x.z;
    a.w2 = x.w2;
    a.gbias = x.gbias;
    a.inv_tau = x.inv_tau;
    a.gtab_off = (int)gate_tab_offset(p.rk);
    // the planned variant must have code for every part the call has
    if ((p.var == kLowRank) != (x.z != nullptr)) return hipErrorInvalidValue;
    if (p.var == kPlain && (x.init || x.gate)) return hipErrorInvalidValue;
    a.q = (const __half*)q;
    a.k = (const __half*)k;
    a.v = (const __half*)v;
    a.lg = (const __half*)lg;
    a.out = (__half*)out;
    a.final_state = final_state;
    unsigned char* base = (unsigned char*)ws;
    const size_t slots = (size_t)p.seq_batch * p.n_spans;
    a.hdr = (unsigned int*)base;
    a.layout = fused_layout_word(p);
    a.fault = g_fault.load(std::memory_order_relaxed);
    a.wait_ticks = (unsigned long long)g_wait_us.load(std::memory_order_relaxed) *
                   wall_ticks_per_ms() / 1000ull;
    a.epoch = (unsigned int*)(base + 256);
    a.agg = (unsigned int*)(base + 256 + align256(slots * sizeof(unsigned int)));
    a.sin = a.agg + (size_t)p.seq_batch * agg_seq_words(p.n_spans);
    a.park = park_bytes(p) ? (u4*)(base + fused_workspace_bytes(s, p) - park_bytes(p)) : nullptr;
    a.L = s.L;
    a.H = s.H;
    a.grid_h = s.grid_h;
    a.grid_w = s.grid_w;
    a.dir = s.dir;
    a.n_chunks = s.n_chunks;
    a.span = p.span;
    a.n_spans = p.n_spans;
    a.slice_log2 = p.slice_log2;
    a.dk = s.d_k;
    a.scale = s.scale;
    if (p.keep && !p.rk && p.span >= 2 && a.park == nullptr) return hipErrorInvalidValue;
    if (p.rk && !rk_span_ok(p.span)) return hipErrorInvalidValue;
    const void* fn = pick_kernel(p.span, p.keep, p.rk, p.var);
    resident_per_cu(p.span, p.keep, p.rk, p.var);   // also raises the kernel's dynamic LDS limit
    const int n_seq = s.B * s.H;
    for (int s0 = 0; s0 < n_seq; s0 += p.seq_batch) {
        a.seq0 = s0;
        const int nseq = (n_seq - s0 < p.seq_batch) ? (n_seq - s0) : p.seq_batch;
        void* args[] = {&a};
        const hipError_t e = hipLaunchKernel(fn, dim3(nseq * p.n_spans), dim3(kThreads), args,
                                             smem_bytes(p.rk, p.var), st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace gtrgla
