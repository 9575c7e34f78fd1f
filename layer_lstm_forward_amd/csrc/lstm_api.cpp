// lstm_api.cpp -- the C ABI declared in include/lstm.h: argument validation,
// workspace carve-up, the per-layer schedule and the kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "../../include/lstm.h"
#include "kernels.h"
#include "pack.h"

using namespace lstm_amd;

struct lstm_plan {
    int I, H, L, D, has_bias, dtype;
    int rec_mode;  // lstm_recurrence
    int rec_tile;  // 0 = automatic, else 100*WK + 10*MTW + NT
    int part_bufs;   // partial-sum buffers requested (1 or 2)
    int poll_sleep;  // back-off between re-reads of stale exchange words
    int read_pace_ns;  // delay between the end of a recurrent step and the first read of the next (-1: by schedule)
    int layer_pipe;    // 1 (default): run a unidirectional stack's layers in one wavefront launch when it fits;
                       // 2: the same with a two-layer stack's layers paired in each workgroup
    int fuse_input;    // 1: compute x_t W_ih^T inside the persistent recurrence when W_ih fits in registers
    int batch_first;   // 1: x and y are [B, T, .] instead of [T, B, .]
    int small_batch;   // 1: B <= 16 layers run each direction's recurrence on one XCD (rec_xcd.hip)
    int resident;      // 1: large-batch layers that would step hold W_hh once across the chip (rec_res.hip); 2: always
    int mode;          // LSTM_MODE_*
    int NG;            // gate blocks of H rows: 4 (LSTM), 3 (GRU), 1 (RNN)
    // training dropout between layers (lstm_set_dropout)
    double dropout;                 // probability, 0 = none
    unsigned long long drop_seed;   // generator key
    unsigned long long drop_call;   // call index of the next lstm_forward_train
                       // (off by default: slower than layer by layer on the measured workloads)
    int team_rows;   // 0 = as many batch rows per team as the tile holds, else at most this many
    int proj_tile;   // projection GEMM (LSTM_OPT_PROJ_TILE): 0 automatic, 1..5 forced
    // optional per-phase timing (LSTM_OPT_TIMING)
    int timing;
    struct Span {
        hipEvent_t a, b;
        int phase;     // 0 projection, 1 recurrence, 2 backward recurrent product, 3 backward gradient product
        int launches;
    };
    std::vector<Span> spans;
    std::vector<hipEvent_t> pool;
    lstm_timing acc;
};

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kStatusBytes = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
bool use_persistent_for_mode(const lstm_plan *p, int B, bool wide);
size_t elem_size(int dtype) { return dtype == LSTM_BF16 ? 2 : 4; }

// Checked products; false on size_t overflow.
bool mul_ok(size_t a, size_t b, size_t *out) {
    if (a != 0 && b > SIZE_MAX / a) return false;
    *out = a * b;
    return true;
}

struct Layout {
    size_t status, xbuf, G, ymid[2], cstate, hstate, lens, wpad, total;
    size_t sync_bytes;  // status word + exchange buffer, zeroed per call
};

// The layer wavefront (rec_wave.hip) applies to unidirectional LSTM stacks of
// 2..kMaxPipeLayers layers in the time-major layout, in a persistent mode with
// its option and the fused input projection on (it computes every input
// product in its launch), whose W_hh and layer-0 input widths fit its tiles.
bool wave_candidate(const lstm_plan *p) {
    int ncx0 = 0;
    return p->layer_pipe && p->fuse_input && p->mode == LSTM_MODE_LSTM && p->D == 1 && p->L >= 2 &&
           p->L <= kMaxPipeLayers &&
           !p->batch_first && (p->rec_mode == LSTM_REC_AUTO || p->rec_mode == LSTM_REC_PERSISTENT) &&
           wave_shape_ok(p->H, p->I, p->dtype, &ncx0);
}

// Teams of the wavefront: at most 16 batch rows each.
int wave_teams(int B) { return (B + 15) / 16; }

// Padded parameters of the GRU and the RNNs, per (layer, direction): W_ih
// [4H][in_l], W_hh [4H][H], b_ih [4H], b_hh [4H] (dtype), each 256-byte
// aligned; fn(l, d, k, offset, rows of the original, columns) for each.
template <class F>
bool walk_padded_params(const lstm_plan *p, F fn) {
    const size_t es = elem_size(p->dtype), G4 = (size_t)4 * p->H;
    size_t off = 0;
    for (int l = 0; l < p->L; ++l)
        for (int d = 0; d < p->D; ++d) {
            const size_t cols[4] = {(size_t)(l == 0 ? p->I : p->D * p->H), (size_t)p->H, 1, 1};
            for (int k = 0; k < 4; ++k) {
                size_t b;
                if (!mul_ok(G4 * cols[k], es, &b) || b > SIZE_MAX / 4 - off) return false;
                fn(l, d, k, off, cols[k]);
                off += align_up(b);
            }
        }
    return true;
}

bool padded_params_bytes(const lstm_plan *p, size_t *bytes) {
    size_t last = 0, last_cols = 0;
    const bool ok = walk_padded_params(p, [&](int, int, int, size_t off, size_t cols) {
        last = off;
        last_cols = cols;
    });
    if (!ok) return false;
    *bytes = last + align_up((size_t)4 * p->H * last_cols * elem_size(p->dtype));
    return true;
}

bool make_layout(const lstm_plan *p, int T, int B, Layout *o) {
    size_t tb, g, y, st, xb;
    if (!mul_ok((size_t)T, (size_t)B, &tb)) return false;
    // exchange tags are l*(T+1) + s + 1 and must fit in 32 bits
    if ((unsigned long long)p->L * ((unsigned long long)T + 1) >= 0xFFFFFFFFull) return false;
    // exchange buffer: 2 parities x D directions x (padded team rows / 16)
    // row tiles x kch chunks x 256 words; padded rows of all teams together
    // never exceed B + 255
    const size_t kch = (size_t)(p->H + (p->dtype == LSTM_BF16 ? 31 : 15)) / (p->dtype == LSTM_BF16 ? 32 : 16);
    if (!mul_ok((size_t)2 * p->D * (((size_t)B + 255) / 16 + 1), kch * 256 * sizeof(unsigned long long), &xb))
        return false;
    // G is [T*B][D][4H] for every mode: the GRU and the RNNs use it with
    // their gate blocks padded to four when they run on the persistent kernel
    if (!mul_ok(tb, (size_t)p->D * 4 * p->H * sizeof(float), &g)) return false;
    // The layer wavefront has no G (every input product runs in its launch)
    // and keeps its exchange words in G's place: one slot per step for every
    // layer but the last, which keeps two; a slot holds kch * 256 32-bit
    // words per team.
    if (wave_candidate(p)) {
        size_t slots, wb;
        if (!mul_ok((size_t)T, (size_t)(p->L - 1), &slots) || !mul_ok(slots + 2, (size_t)wave_teams(B), &slots) ||
            !mul_ok(slots, kch * 256 * sizeof(uint32_t), &wb))
            return false;
        if (wb > g) g = wb;
    }
    if (!mul_ok(tb, (size_t)p->D * p->H * elem_size(p->dtype), &y)) return false;
    if (!mul_ok((size_t)p->D * B, (size_t)p->H * sizeof(float), &st)) return false;
    size_t off = 0;
    o->status = off;
    off += kStatusBytes;
    o->xbuf = off;
    off += align_up(xb);
    o->sync_bytes = off;
    o->G = off;
    if (g > SIZE_MAX / 2) return false;
    off += align_up(g);
    const int nmid = p->L >= 3 ? 2 : (p->L == 2 ? 1 : 0);
    for (int i = 0; i < 2; ++i) {
        o->ymid[i] = off;
        if (i < nmid) off += align_up(y);
    }
    o->cstate = off;
    off += align_up(st);
    o->hstate = off;  // h carry of stepped launches with per-row lengths
    off += align_up(st);
    o->lens = off;    // per-row lengths, copied from the caller's host array
    off += align_up((size_t)B * sizeof(int));
    o->wpad = off;    // the GRU's and the RNNs' parameters padded to four gate blocks
    if (p->mode != LSTM_MODE_LSTM) {
        size_t wp = 0;
        if (!padded_params_bytes(p, &wp)) return false;
        off += wp;
    }
    o->total = off;
    return true;
}

// Training reserve: per layer the activations [T][B][D][5][H] fp32 (gates i,
// f, g, o and c of every step), then the outputs of the layers below the top
// one ([T][B][D*H] dtype) that the backward pass reads again; with dropout,
// per layer below the top one also the next layer's input (the output after
// dropout, dtype) and the keep decisions (one byte per element).
struct ReserveLayout {
    size_t acts_layer, y_layer, xd_layer, keep_layer, total;
    bool dropout;
    // layer l's output (l < L - 1), the next layer's input after dropout, and the keep bytes
    size_t y(const lstm_plan *p, int l) const { return acts_layer * p->L + y_layer * l; }
    size_t xd(const lstm_plan *p, int l) const {
        return acts_layer * p->L + y_layer * (p->L - 1) + (xd_layer + keep_layer) * l;
    }
    size_t keep(const lstm_plan *p, int l) const { return xd(p, l) + xd_layer; }
};

bool make_reserve(const lstm_plan *p, int T, int B, ReserveLayout *r) {
    size_t tb, a, y;
    if (T < 1 || B < 1 || !mul_ok((size_t)T, (size_t)B, &tb)) return false;
    if (!mul_ok(tb, (size_t)p->D * 5 * p->H * sizeof(float), &a)) return false;
    if (!mul_ok(tb, (size_t)p->D * p->H * elem_size(p->dtype), &y)) return false;
    r->acts_layer = align_up(a);
    r->y_layer = align_up(y);
    r->dropout = p->dropout > 0.0 && p->L > 1;
    r->xd_layer = r->dropout ? r->y_layer : 0;
    r->keep_layer = r->dropout ? align_up(y / elem_size(p->dtype)) : 0;
    size_t ta, ty, td;
    if (!mul_ok(r->acts_layer, (size_t)p->L, &ta) || !mul_ok(r->y_layer, (size_t)(p->L - 1), &ty) ||
        !mul_ok(r->xd_layer + r->keep_layer, (size_t)(p->L - 1), &td))
        return false;
    if (ta > SIZE_MAX - ty || ta + ty > SIZE_MAX - td) return false;
    r->total = ta + ty + td;
    return true;
}

// Backward workspace (all fp32): dz [T][B][D][4H]; one direction's dz^T
// [4H][T*B]; the layer input x^T [in][T*B] and h_prev^T [H][T*B]; two output
// gradient buffers [T*B][max(in, D*H)] (this layer's dY and the dX it
// produces); the cell gradient carry and dh_n [D][B][H]; transposed W_hh
// [D][H][4H] and W_ih [in][D*4H]; the K-split slabs of the gradient products;
// one bias gradient [4H].
struct BwdLayout {
    size_t status, pbuf, dz, dzt, xt, ht, dy[2], dc, dhn, wht, wcat, ksp, db, lens, dhc, total;
};

// row chunks of the bias-gradient column sums
constexpr int kBiasChunks = 128;

// K-split count of an fp32 M x N x K product (1: not split)
int ksplit_count(int M, int N, int K) {
    const int kc = proj_kchunk(M, N, K);
    return kc ? (K + kc - 1) / kc : 1;
}

bool make_bwd_layout(const lstm_plan *p, int T, int B, BwdLayout *o) {
    if (T < 1 || B < 1) return false;
    const size_t G4 = (size_t)4 * p->H, H = p->H, D = p->D, f = sizeof(float);
    const size_t win = std::max((size_t)p->I, D * H);
    size_t tb;
    if (!mul_ok((size_t)T, (size_t)B, &tb) || tb > (size_t)INT_MAX) return false;
    size_t sz[16];
    sz[14] = kStatusBytes;  // status word first, as in the forward's workspace
    // partial sums handed between the two halves of a K-split backward step
    sz[15] = D * (size_t)((B + 15) / 16) * ((H + 15) / 16) * 256 * sizeof(unsigned long long);
    if (!mul_ok(tb, D * G4 * f, &sz[0]) || !mul_ok(tb, G4 * f, &sz[1]) || !mul_ok(tb, win * f, &sz[2]) ||
        !mul_ok(tb, H * f, &sz[3]) || !mul_ok(tb, win * f, &sz[4]))
        return false;
    sz[5] = sz[4];
    sz[6] = D * B * H * f;
    sz[7] = sz[6];
    sz[8] = D * H * G4 * f;
    sz[9] = win * D * G4 * f;
    // K-split slabs (or the unsplit fp32 product) of the weight-gradient
    // products, and the slabs of a split input-gradient product
    size_t ksp = 0;
    for (int l = 0; l < p->L; ++l) {
        const int in_l = l == 0 ? p->I : (int)(D * H);
        const size_t kw = std::max((size_t)ksplit_count((int)G4, in_l, (int)tb) * in_l,
                                   (size_t)ksplit_count((int)G4, (int)H, (int)tb) * H) * G4;
        ksp = std::max(ksp, kw);
        const int nx = ksplit_count((int)tb, in_l, (int)(D * G4));
        if (nx > 1) ksp = std::max(ksp, (size_t)nx * tb * in_l);
    }
    if (!mul_ok(ksp, f, &sz[10])) return false;
    sz[11] = (size_t)kBiasChunks * G4 * f;  // bias-gradient partial sums
    sz[12] = (size_t)B * sizeof(int);        // per-row lengths
    sz[13] = D * B * H * f;                  // gradient of h carried through padded steps
    size_t *dst[16] = {&o->dz, &o->dzt, &o->xt, &o->ht, &o->dy[0], &o->dy[1], &o->dc, &o->dhn,
                       &o->wht, &o->wcat, &o->ksp, &o->db, &o->lens, &o->dhc, &o->status, &o->pbuf};
    const int order[16] = {14, 15, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13};
    size_t off = 0;
    for (int i : order) {
        *dst[i] = off;
        if (sz[i] > SIZE_MAX - off - 256) return false;
        off += align_up(sz[i]);
    }
    o->total = off;
    return true;
}

// ---------------------------------------------------------------- schedule
struct Sched {
    bool persistent;
    bool wide;  // bf16 exchange in wide words (one value per word)
    RecTile tile;
    RecGeom geom;
    int U, P, BG, NGB, teams, wgs, map_xcd;
    size_t smem;
};

// The read pace of a persistent schedule (LSTM_OPT_READ_PACE unless set).
// A read of the others' h_t that reaches memory before the data costs a
// retry round trip, one that waits too long idles.  Measured optima: 450 ns
// when one team spans every XCD (P = 256: the latency-bound B = 1 and 4
// workloads), ~375 ns for 8-unit slices (the fp32 benchmark, 0.991 -> 0.975
// ms against 450), ~300 ns for 16-unit slices, whose own step is longer (the
// bidirectional bf16 workload, 1.742 -> 1.674 ms).
int read_pace_for(const lstm_plan *p, const Sched &s) {
    if (p->read_pace_ns >= 0) return p->read_pace_ns;
    if (s.P >= 256) return 450;
    return s.U >= 16 ? 300 : 375;
}

struct DevInfo {
    bool ok;
    int cus;
    int wall_khz;
};

DevInfo dev_info(int dev) {
    static std::mutex mu;
    static DevInfo cache[64];
    static bool have[64];
    std::lock_guard<std::mutex> g(mu);
    if (dev < 0 || dev >= 64) return DevInfo{false, 0, 0};
    if (!have[dev]) {
        DevInfo d{true, 0, 0};
        if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipDeviceGetAttribute(&d.wall_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
            d.ok = false;
        if (d.wall_khz <= 0) d.wall_khz = 100000;
        cache[dev] = d;
        have[dev] = d.ok;
        return d;
    }
    return cache[dev];
}

const RecTile kTiles[] = {{4, 1, 4}, {4, 1, 2}, {4, 1, 1}, {2, 1, 4}, {2, 1, 2}, {2, 1, 1},
                          {1, 1, 4}, {1, 1, 2}, {1, 1, 1}, {1, 4, 2}, {1, 4, 1}};

bool fill_sched(const lstm_plan *p, int B, RecTile t, Sched *s) {
    if (!rec_tile_supported(t)) return false;
    const int rows = rec_rows_per_wg(t);
    s->tile = t;
    s->U = 4 * t.NT;
    s->P = (p->H + s->U - 1) / s->U;
    const int cap = p->team_rows > 0 && p->team_rows < rows ? p->team_rows : rows;
    const int ng0 = (B + cap - 1) / cap;
    s->BG = (B + ng0 - 1) / ng0;
    s->NGB = (B + s->BG - 1) / s->BG;
    s->teams = s->NGB * p->D;
    s->wgs = s->teams * s->P;
    s->geom = rec_geom(t, p->H, p->dtype, p->part_bufs == 2);
    s->smem = s->geom.smem;
    s->map_xcd = (s->teams <= 8 && 8 % s->teams == 0 && (s->wgs % 8) == 0) ? 1 : 0;
    // the exchange buffer (make_layout) holds (B + 255) / 16 + 1 row tiles of
    // 8-byte words per direction and parity, i.e. that many tiles of wide
    // words: the teams' padded row tiles must fit (a small LSTM_OPT_TEAM_ROWS
    // makes many teams of mostly padding rows)
    const bool fits_xbuf = (size_t)s->NGB * (rows / 16) <= ((size_t)B + 255) / 16 + 1;
    return fits_xbuf && s->teams <= kMaxTeams && s->smem <= kRecLdsLimit;
}

// bf16 recurrences whose exchanged h may reach 2 in magnitude take the wide
// exchange words: the relu RNN (unbounded), the GRU from a caller's h0 (h
// moves from h0 towards values in [-1, 1] without a bound of 1), and per-row
// lengths with a caller's h0 (the reverse scan republishes h0 on its leading
// padded steps).  The LSTM's o tanh(c) and the tanh RNN's output are bounded
// by 1 otherwise.
bool needs_wide_exchange(const lstm_plan *p, bool have_h0, bool have_lengths) {
    if (p->dtype != LSTM_BF16) return false;
    return p->mode == LSTM_MODE_RNN_RELU || (have_h0 && (p->mode == LSTM_MODE_GRU || have_lengths));
}

// Rough cycles per step of one workgroup: matrix-core work of the busiest
// wave (times the number of workgroups that share a CU), plus the h_{t-1}
// fetch as tagged 32-bit words (one fp32 or two bf16 values each) at the
// ~32 B/clk a CU sustains for it.
double step_cost(const lstm_plan *p, const Sched &s, int cus) {
    const int kc = p->dtype == LSTM_BF16 ? 32 : 16;
    const int kch = (p->H + kc - 1) / kc;
    const int cpw = (kch + s.tile.WK - 1) / s.tile.WK;
    const int live_mtw = (s.BG + 15) / 16 < s.tile.MTW ? (s.BG + 15) / 16 : s.tile.MTW;
    const int share = cus > 0 ? (s.wgs + cus - 1) / cus : 1;
    const double mfma = (double)live_mtw * s.tile.NT * cpw * (p->dtype == LSTM_BF16 ? 16 : 128) * share;
    const double xbytes = (double)s.BG * p->H * (p->dtype == LSTM_BF16 ? 2 : 4) * share;
    return mfma + xbytes / 32.0;
}

// Input chunks per wave when layer input X (width in_l) can use the fused
// projection of the chosen persistent schedule, else 0: the tile has a fused
// variant whose register budget covers the wave's share of the input width,
// rows are 16-byte multiples and aligned, one time slice of X is addressable
// by a buffer resource, and the fused kernel is co-resident like the plain one.
int fused_chunks_shape(const lstm_plan *p, const Sched &s, int T, int B, int in_l, const DevInfo &di) {
    if (!p->fuse_input || !s.persistent || !s.geom.wreg || !di.ok) return 0;
    const int fx = rec_fused_chunks(s.tile);
    if (fx == 0) return 0;
    const size_t es = elem_size(p->dtype);
    const int kc = p->dtype == LSTM_BF16 ? 32 : 16;
    const int ncx = ((in_l + kc - 1) / kc + s.tile.WK - 1) / s.tile.WK;
    // one buffer resource spans the B rows of one time step: B rows in a row
    // (time-major) or T rows apart (batch_first)
    const size_t span = (size_t)B * in_l * es * (p->batch_first ? (size_t)T : 1);
    if (ncx > fx || ((size_t)in_l * es) % 16 != 0 || span >= ((size_t)1 << 31)) return 0;
    return ncx;
}

int fused_chunks(const lstm_plan *p, const Sched &s, int T, int B, int in_l, const void *X,
                 const void *const *wih, const DevInfo &di) {
    const int ncx = fused_chunks_shape(p, s, T, B, in_l, di);
    if (ncx == 0 || (uintptr_t)X % 16 != 0) return 0;
    for (int d = 0; d < p->D; ++d)
        if ((uintptr_t)wih[d] % 16 != 0) return 0;
    int bpc = 0;
    const bool fits = rec_max_coresident(s.tile, s.smem, p->dtype, true, true, s.wide, &bpc) == hipSuccess && bpc > 0 &&
                      (long long)bpc * di.cus >= s.wgs;
    (void)hipGetLastError();
    return fits ? ncx : 0;
}

int choose_sched(const lstm_plan *p, int B, int dev, Sched *out, bool wide) {
    const DevInfo di = dev_info(dev);
    Sched best{};
    double best_cost = 1e300;
    bool found = false;
    const bool want_step = p->rec_mode == LSTM_REC_STEP || p->rec_mode == LSTM_REC_GEMM;
    for (const RecTile &t : kTiles) {
        if (p->rec_tile && p->rec_tile != 100 * t.WK + 10 * t.MTW + t.NT) continue;
        Sched s{};
        if (!fill_sched(p, B, t, &s)) continue;
        s.wide = wide;
        bool can_persist = false;
        if (!want_step && di.ok) {
            int bpc = 0;
            if (rec_max_coresident(t, s.smem, p->dtype, s.geom.wreg != 0, false, wide, &bpc) == hipSuccess && bpc > 0)
                can_persist = (long long)bpc * di.cus >= s.wgs;
            (void)hipGetLastError();
        }
        if (p->rec_mode == LSTM_REC_PERSISTENT && !can_persist) continue;
        s.persistent = can_persist;
        double cost;
        if (s.persistent) {
            cost = step_cost(p, s, di.cus);
        } else {
            // per step launch: every workgroup reloads its W_hh slice
            cost = 1e12 + (double)s.wgs * (4.0 * s.U + s.BG) * p->H * elem_size(p->dtype);
        }
        if (cost < best_cost) {
            best_cost = cost;
            best = s;
            found = true;
        }
    }
    if (!found) return LSTM_ERR_UNSUPPORTED;
    *out = best;
    return LSTM_OK;
}

// Shape conditions of the per-step GEMM kernel (k_rec_step); pointer
// alignment is checked per call.
bool gemm_step_shape_ok(const lstm_plan *p) {
    const size_t es = elem_size(p->dtype);
    return p->rec_mode != LSTM_REC_STEP && ((size_t)p->H * es) % 16 == 0 &&
           (size_t)4 * p->H * p->H * es < (1u << 31) && (size_t)128 * p->D * p->H * es < (1u << 31);
}

struct WaveSched {
    int NT, U, P, BG, NGB, wgs, ncx0, map_xcd;
    int lpw;  // layers per workgroup: 1, or 2 (a two-layer stack paired in 512-thread workgroups)
};

// Wavefront schedule: teams of at most 16 rows, U = 4 NT units per
// workgroup; every (layer, team, unit slice) workgroup must be co-resident.
// The smallest NT that fits spreads the work over the most workgroups.
bool choose_wave(const lstm_plan *p, int B, int dev, WaveSched *out) {
    if (!wave_candidate(p)) return false;
    const DevInfo di = dev_info(dev);
    if (!di.ok) return false;
    for (int nt = 1; nt <= 4; nt *= 2) {
        if (p->rec_tile && p->rec_tile != 410 + nt) continue;
        WaveSched w{};
        w.NT = nt;
        w.U = 4 * nt;
        w.P = (p->H + w.U - 1) / w.U;
        w.NGB = wave_teams(B);
        w.BG = (B + w.NGB - 1) / w.NGB;
        w.lpw = (p->layer_pipe == 2 && p->L == 2 && nt <= 2) ? 2 : 1;
        w.wgs = (w.lpw == 2 ? 1 : p->L) * w.NGB * w.P;
        wave_shape_ok(p->H, p->I, p->dtype, &w.ncx0);
        const int per_layer = w.NGB * w.P;
        w.map_xcd = (w.NGB <= 8 && 8 % w.NGB == 0 && per_layer % 8 == 0) ? 1 : 0;
        int bpc = 0;
        const bool ok = wave_max_coresident(nt, p->dtype, w.lpw, &bpc) == hipSuccess && bpc > 0 &&
                        (long long)bpc * di.cus >= w.wgs;
        (void)hipGetLastError();
        if (ok) {
            *out = w;
            return true;
        }
    }
    return false;
}

// The small-batch recurrence (rec_xcd.hip): time-major LSTM inference with
// B <= 16 whose W_hh fits one XCD's registers, all its workgroups co-resident.
bool use_xcd(const lstm_plan *p, int B, int dev) {
    if (!p->small_batch || p->mode != LSTM_MODE_LSTM || p->batch_first ||
        !(p->rec_mode == LSTM_REC_AUTO || p->rec_mode == LSTM_REC_PERSISTENT) || p->rec_tile != 0 ||
        !xcd_shape_ok(p->H, B, p->D, p->dtype))
        return false;
    const DevInfo di = dev_info(dev);
    int bpc = 0;
    const bool ok = di.ok && xcd_max_coresident(p->dtype, &bpc) == hipSuccess && bpc > 0 &&
                    (long long)bpc * di.cus >= 8LL * xcd_workgroups(p->H) && di.cus >= 256;
    (void)hipGetLastError();
    return ok;
}

// The large-batch resident recurrence (rec_res.hip): time-major bf16 LSTM
// inference whose layer would otherwise step (option 1) or always when the
// shape allows (option 2), every workgroup co-resident.
bool use_res(const lstm_plan *p, int B, int dev, bool persistent, int *groups, int *slices, int *map_xcd) {
    if (!p->resident || (p->resident == 1 && persistent) || p->mode != LSTM_MODE_LSTM || p->batch_first ||
        !(p->rec_mode == LSTM_REC_AUTO || p->rec_mode == LSTM_REC_PERSISTENT) || p->rec_tile != 0)
        return false;
    const DevInfo di = dev_info(dev);
    if (!di.ok || !res_shape_ok(p->H, B, p->D, p->dtype, di.cus, groups, slices, map_xcd)) return false;
    int bpc = 0;
    const bool ok = res_max_coresident(p->H, &bpc) == hipSuccess && bpc > 0 &&
                    (long long)bpc * di.cus >= (long long)*groups * *slices;
    (void)hipGetLastError();
    return ok;
}

hipEvent_t take_event(lstm_plan *p) {
    if (!p->pool.empty()) {
        hipEvent_t e = p->pool.back();
        p->pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    return e;
}

// Record the start of a timed span on `st`; returns the span index or -1.
int span_begin(lstm_plan *p, hipStream_t st, int phase) {
    if (!p->timing) return -1;
    lstm_plan::Span sp{take_event(p), take_event(p), phase, 0};
    if (!sp.a || !sp.b || hipEventRecord(sp.a, st) != hipSuccess) {
        (void)hipGetLastError();
        if (sp.a) p->pool.push_back(sp.a);
        if (sp.b) p->pool.push_back(sp.b);
        return -1;
    }
    p->spans.push_back(sp);
    return (int)p->spans.size() - 1;
}

void span_end(lstm_plan *p, int idx, hipStream_t st, int launches) {
    if (idx < 0) return;
    p->spans[idx].launches = launches;
    if (hipEventRecord(p->spans[idx].b, st) != hipSuccess) (void)hipGetLastError();
}

bool is_device_ptr(const void *ptr, int dev) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    if (hipPointerGetAttributes(&attr, ptr) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    const bool dev_mem = attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
    return dev_mem && attr.device == dev;
}

int validate(const lstm_plan *p, const void *x, const void *h0, const float *c0,
             const void *const *weights, int T, int B, int layers, int bidir, const void *y,
             const void *ws, size_t ws_bytes, Layout *lay) {
    if (!p) return LSTM_ERR_ARG;
    if (layers != p->L || (bidir ? 2 : 1) != p->D || (bidir != 0 && bidir != 1)) return LSTM_ERR_SHAPE;
    if (T < 1 || B < 1) return LSTM_ERR_SHAPE;
    if ((long long)T * B > INT_MAX) return LSTM_ERR_SHAPE;
    if (!x || !y || !weights) return LSTM_ERR_ARG;
    // the LSTM's initial state is a pair; the other modes have no cell state
    if (p->mode == LSTM_MODE_LSTM ? (h0 == nullptr) != (c0 == nullptr) : c0 != nullptr) return LSTM_ERR_ARG;
    const int per = p->has_bias ? 4 : 2;
    for (int i = 0; i < p->L * p->D * per; ++i)
        if (!weights[i]) return LSTM_ERR_ARG;
    if (!make_layout(p, T, B, lay)) return LSTM_ERR_SHAPE;
    if (!ws || ws_bytes < lay->total) return LSTM_ERR_WORKSPACE;
    return LSTM_OK;
}

}  // namespace

extern "C" {

int lstm_version(void) { return 110; }

const char *lstm_strerror(int s) {
    switch (s) {
        case LSTM_OK: return "ok";
        case LSTM_ERR_ARG: return "invalid argument (NULL pointer, non-positive size, or h0/c0 not given together)";
        case LSTM_ERR_SHAPE: return "invalid shape (T or B < 1, layers/bidir differ from the plan, or size overflow)";
        case LSTM_ERR_DTYPE: return "unknown dtype";
        case LSTM_ERR_DEVICE: return "pointer is not device memory of the current device, or no device";
        case LSTM_ERR_WORKSPACE: return "workspace missing or smaller than lstm_workspace_size";
        case LSTM_ERR_LAUNCH: return "kernel launch failed";
        case LSTM_ERR_UNSUPPORTED: return "unsupported option or schedule";
        case LSTM_ERR_DEVICE_TIMEOUT: return "a step barrier timed out on the device; outputs are invalid";
        default: return "unknown status";
    }
}

lstm_status lstm_create(lstm_plan **out, int input_size, int hidden_size, int num_layers,
                        int bidirectional, int has_bias, int dtype) {
    return lstm_create_mode(out, LSTM_MODE_LSTM, input_size, hidden_size, num_layers, bidirectional, has_bias,
                            dtype);
}

lstm_status lstm_create_mode(lstm_plan **out, int mode, int input_size, int hidden_size, int num_layers,
                             int bidirectional, int has_bias, int dtype) {
    if (!out) return LSTM_ERR_ARG;
    *out = nullptr;
    if (mode < LSTM_MODE_LSTM || mode > LSTM_MODE_RNN_RELU) return LSTM_ERR_ARG;
    if (dtype != LSTM_F32 && dtype != LSTM_BF16) return LSTM_ERR_DTYPE;
    if (input_size < 1 || hidden_size < 1 || num_layers < 1) return LSTM_ERR_ARG;
    if ((bidirectional != 0 && bidirectional != 1) || (has_bias != 0 && has_bias != 1)) return LSTM_ERR_ARG;
    // 4H and D*4H index rows and columns as int in the kernels
    if ((long long)hidden_size * 8 > INT_MAX / 4) return LSTM_ERR_SHAPE;
    lstm_plan *p = new (std::nothrow) lstm_plan;
    if (!p) return LSTM_ERR_ARG;
    p->I = input_size;
    p->H = hidden_size;
    p->L = num_layers;
    p->D = bidirectional ? 2 : 1;
    p->has_bias = has_bias;
    p->dtype = dtype;
    p->rec_mode = LSTM_REC_AUTO;
    p->rec_tile = 0;
    p->part_bufs = 1;
    p->poll_sleep = 2;
    p->read_pace_ns = -1;
    p->layer_pipe = 1;
    p->fuse_input = 1;
    p->batch_first = 0;
    p->small_batch = 1;
    p->resident = 1;
    p->mode = mode;
    p->NG = mode == LSTM_MODE_LSTM ? 4 : mode == LSTM_MODE_GRU ? 3 : 1;
    p->dropout = 0.0;
    p->drop_seed = 0;
    p->drop_call = 0;
    p->team_rows = 0;
    p->proj_tile = 0;
    p->timing = 0;
    p->acc = lstm_timing{};
    *out = p;
    return LSTM_OK;
}

void lstm_destroy(lstm_plan *p) {
    if (!p) return;
    for (auto &sp : p->spans) {
        (void)hipEventSynchronize(sp.b);
        (void)hipEventDestroy(sp.a);
        (void)hipEventDestroy(sp.b);
    }
    for (hipEvent_t e : p->pool) (void)hipEventDestroy(e);
    (void)hipGetLastError();
    delete p;
}

lstm_status lstm_read_timing(lstm_plan *p, lstm_timing *out, int reset) {
    if (!p || !out) return LSTM_ERR_ARG;
    for (auto &sp : p->spans) {
        float ms = 0.f;
        if (hipEventSynchronize(sp.b) == hipSuccess && hipEventElapsedTime(&ms, sp.a, sp.b) == hipSuccess) {
            if (sp.phase == 0) {
                p->acc.proj_ms += ms;
                p->acc.proj_launches += sp.launches;
            } else if (sp.phase == 1) {
                p->acc.rec_ms += ms;
                p->acc.rec_launches += sp.launches;
            } else if (sp.phase == 2) {
                p->acc.bwd_rec_ms += ms;
                p->acc.bwd_rec_launches += sp.launches;
            } else {
                p->acc.bwd_gemm_ms += ms;
                p->acc.bwd_gemm_launches += sp.launches;
            }
        } else {
            (void)hipGetLastError();
        }
        p->pool.push_back(sp.a);
        p->pool.push_back(sp.b);
    }
    p->spans.clear();
    *out = p->acc;
    if (reset) p->acc = lstm_timing{};
    return LSTM_OK;
}

lstm_status lstm_set_dropout(lstm_plan *p, double prob, unsigned long long seed, unsigned long long call) {
    if (!p || !(prob >= 0.0 && prob <= 1.0)) return LSTM_ERR_ARG;
    p->dropout = prob;
    p->drop_seed = seed;
    p->drop_call = call;
    return LSTM_OK;
}

lstm_status lstm_set_option(lstm_plan *p, int option, int value) {
    if (!p) return LSTM_ERR_ARG;
    switch (option) {
        case LSTM_OPT_RECURRENCE:
            if (value < LSTM_REC_AUTO || value > LSTM_REC_GEMM) return LSTM_ERR_UNSUPPORTED;
            p->rec_mode = value;
            return LSTM_OK;
        case LSTM_OPT_PARTIAL_BUFFERS:
            if (value != 1 && value != 2) return LSTM_ERR_UNSUPPORTED;
            p->part_bufs = value;
            return LSTM_OK;
        case LSTM_OPT_POLL_SLEEP:
            if (value < 0 || value > 1000) return LSTM_ERR_UNSUPPORTED;
            p->poll_sleep = value;
            return LSTM_OK;
        case LSTM_OPT_LAYER_PIPE:
            if (value < 0 || value > 2) return LSTM_ERR_UNSUPPORTED;
            p->layer_pipe = value;
            return LSTM_OK;
        case LSTM_OPT_FUSE_INPUT:
            if (value != 0 && value != 1) return LSTM_ERR_UNSUPPORTED;
            p->fuse_input = value;
            return LSTM_OK;
        case LSTM_OPT_BATCH_FIRST:
            if (value != 0 && value != 1) return LSTM_ERR_UNSUPPORTED;
            p->batch_first = value;
            return LSTM_OK;
        case LSTM_OPT_SMALL_BATCH:
            if (value != 0 && value != 1) return LSTM_ERR_UNSUPPORTED;
            p->small_batch = value;
            return LSTM_OK;
        case LSTM_OPT_RESIDENT:
            if (value < 0 || value > 2) return LSTM_ERR_UNSUPPORTED;
            p->resident = value;
            return LSTM_OK;
        case LSTM_OPT_READ_PACE:
            if (value < 0 || value > 100000) return LSTM_ERR_UNSUPPORTED;
            p->read_pace_ns = value;
            return LSTM_OK;
        case LSTM_OPT_TEAM_ROWS:
            if (value < 0) return LSTM_ERR_UNSUPPORTED;
            p->team_rows = value;
            return LSTM_OK;
        case LSTM_OPT_PROJ_TILE:
            if (value < 0 || value > 7) return LSTM_ERR_UNSUPPORTED;
            p->proj_tile = value;
            return LSTM_OK;
        case LSTM_OPT_TIMING:
            if (value != 0 && value != 1) return LSTM_ERR_UNSUPPORTED;
            p->timing = value;
            return LSTM_OK;
        case LSTM_OPT_REC_TILE:
            if (value != 0 && !rec_tile_supported(RecTile{value / 100, (value / 10) % 10, value % 10}))
                return LSTM_ERR_UNSUPPORTED;
            p->rec_tile = value;
            return LSTM_OK;
        default:
            return LSTM_ERR_UNSUPPORTED;
    }
}

lstm_status lstm_workspace_size(const lstm_plan *p, int T, int B, size_t *bytes) {
    if (!p || !bytes) return LSTM_ERR_ARG;
    if (T < 1 || B < 1) return LSTM_ERR_SHAPE;
    Layout lay;
    if (!make_layout(p, T, B, &lay)) return LSTM_ERR_SHAPE;
    *bytes = lay.total;
    return LSTM_OK;
}

lstm_status lstm_describe(const lstm_plan *p, int T, int B, char *buf, size_t len) {
    if (!p || !buf || len == 0) return LSTM_ERR_ARG;
    if (T < 1 || B < 1) return LSTM_ERR_SHAPE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    const int in0 = p->I > p->D * p->H ? p->I : p->D * p->H;  // widest layer input
    const char *dt = p->dtype == LSTM_BF16 ? "bf16" : "f32";
    static const char *names[] = {"lstm", "gru", "rnn_tanh", "rnn_relu"};
    // (describes a call without h0 or lengths)
    const bool wide = needs_wide_exchange(p, false, false);
    const bool mode_persistent = p->mode != LSTM_MODE_LSTM && use_persistent_for_mode(p, B, wide);
    if (p->mode != LSTM_MODE_LSTM && !mode_persistent) {
        const int bm = rec_step_rows(B);
        std::snprintf(buf, len,
                      "cell=%s proj=%s<%s>; rec=k_rec_step<%s> mode=gemm-step block=%dx32 workgroups=%d launches=T%s",
                      names[p->mode], proj_kernel_name(T * B, p->NG * p->H, in0, p->D, p->dtype, p->proj_tile), dt, dt,
                      bm, ((B + bm - 1) / bm) * ((p->H + 31) / 32) * p->D, p->batch_first ? " layout=batch-first" : "");
        return LSTM_OK;
    }
    Sched s{};
    const int rc = choose_sched(p, B, dev, &s, wide);
    if (rc != LSTM_OK) return (lstm_status)rc;
    const char *proj = proj_kernel_name(T * B, 4 * p->H, in0, p->D, p->dtype, p->proj_tile);
    WaveSched ws{};
    if (!mode_persistent && choose_wave(p, B, dev, &ws)) {
        std::snprintf(buf, len,
                      "rec=k_rec_wave<%s,NT=%d> mode=wavefront U=%d P=%d BG=%d NGB=%d layers=%d layers_per_wg=%d "
                      "workgroups=%d map_xcd=%d w_hh=regs xproj=%s",
                      dt, ws.NT, ws.U, ws.P, ws.BG, ws.NGB, p->L, ws.lpw, ws.wgs, ws.map_xcd,
                      p->L == 2 ? "fused,fused" : p->L == 3 ? "fused,fused,fused" : "fused,fused,fused,fused");
        return LSTM_OK;
    }
    if (!mode_persistent && use_xcd(p, B, dev)) {
        std::snprintf(buf, len, "proj=%s<%s>; rec=k_rec_xcd<%s> mode=small-batch units=32 workgroups=%d per direction "
                      "(one XCD each) w_hh=regs xproj=hoisted",
                      proj, dt, dt, xcd_workgroups(p->H));
        return LSTM_OK;
    }
    int rg = 0, rs = 0, rmap = 0;
    if (!mode_persistent && use_res(p, B, dev, s.persistent, &rg, &rs, &rmap)) {
        std::snprintf(buf, len, "proj=%s<%s>; rec=k_rec_res<%s> mode=resident rows=128 units=16 workgroups=%d "
                      "map_xcd=%d w_hh=regs h_via=ring xproj=hoisted",
                      proj, dt, dt, rg * rs, rmap);
        return LSTM_OK;
    }
    if (!s.persistent && gemm_step_shape_ok(p)) {
        // per-step GEMM (assuming 16-byte aligned operands, as lstm_forward checks)
        const int bm = rec_step_rows(B);
        std::snprintf(buf, len, "proj=%s<%s>; rec=k_rec_step<%s> mode=gemm-step block=%dx32 workgroups=%d launches=T",
                      proj, dt, dt, bm, ((B + bm - 1) / bm) * ((p->H + 31) / 32) * p->D);
        return LSTM_OK;
    }
    // per layer: is the input projection fused into the recurrence (assuming
    // 16-byte aligned operands and a co-resident fused kernel)?
    const DevInfo di = dev_info(dev);
    char xproj[64] = {0};
    size_t xl = 0;
    for (int l = 0; l < p->L && xl + 9 < sizeof(xproj); ++l) {
        const int in_l = l == 0 ? p->I : p->D * p->H;
        xl += (size_t)std::snprintf(xproj + xl, sizeof(xproj) - xl, "%s%s", l ? "," : "",
                                    p->mode != LSTM_MODE_GRU && fused_chunks_shape(p, s, T, B, in_l, di) ? "fused"
                                                                                                       : "hoisted");
    }
    char cell[64] = {0};
    if (mode_persistent) std::snprintf(cell, sizeof(cell), "cell=%s gate_slots=4 ", names[p->mode]);
    std::snprintf(buf, len,
                  "%sproj=%s<%s>; rec=k_rec<%s,WK=%d,MTW=%d,NT=%d> mode=%s U=%d P=%d BG=%d "
                  "NGB=%d teams=%d workgroups=%d lds=%zu partial_bufs=%d map_xcd=%d w_hh=%s xproj=%s xwords=%s%s",
                  cell, proj, dt, dt, s.tile.WK, s.tile.MTW, s.tile.NT, s.persistent ? "persistent" : "step", s.U, s.P,
                  s.BG, s.NGB, s.teams, s.wgs, s.smem, s.geom.part_bufs, s.map_xcd, s.geom.wreg ? "regs" : "lds",
                  xproj, p->dtype != LSTM_BF16 ? "f32" : s.wide ? "wide" : "pair",
                  p->batch_first ? " layout=batch-first" : "");
    return LSTM_OK;
}

}  // extern "C"

namespace {

// The forward pass; lengths_h: NULL (every row has T steps) or B host values
// in 1..T, already validated.
// own_ws: the workspace is the library's own device array (lstm_forward_static),
// not caller memory, and is not checked as one.
lstm_status forward_impl(lstm_plan *p, const void *x, const int *lengths_h, const void *h0, const float *c0,
                         const void *const *weights, int T, int B, int layers, int bidir, void *y,
                         void *h_n, float *c_n, void *workspace, size_t workspace_bytes, void *stream_,
                         char *reserve = nullptr, bool own_ws = false) {
    Layout lay;
    int rc = validate(p, x, h0, c0, weights, T, B, layers, bidir, y, workspace, workspace_bytes, &lay);
    if (rc != LSTM_OK) return (lstm_status)rc;
    ReserveLayout rl{};
    if (reserve && !make_reserve(p, T, B, &rl)) return LSTM_ERR_SHAPE;

    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    const int per = p->has_bias ? 4 : 2;
    const void *ptrs[] = {x, y, own_ws ? nullptr : workspace, h0, c0, h_n, c_n};
    for (const void *q : ptrs)
        if (q && !is_device_ptr(q, dev)) return LSTM_ERR_DEVICE;
    for (int i = 0; i < p->L * p->D * per; ++i)
        if (!is_device_ptr(weights[i], dev)) return LSTM_ERR_DEVICE;

    Sched sch{};
    rc = choose_sched(p, B, dev, &sch, needs_wide_exchange(p, h0 != nullptr, lengths_h != nullptr));
    if (rc != LSTM_OK) return (lstm_status)rc;
    const DevInfo di = dev_info(dev);

    hipStream_t st = static_cast<hipStream_t>(stream_);
    char *ws = static_cast<char *>(workspace);

    // The GRU and the plain RNNs run on the LSTM's four gate slots: their
    // parameters are copied with zero rows up to four gate blocks (the GRU's
    // b_hh keeps only its r and z blocks: b_hn is added inside the reset
    // product by the kernel, from the caller's b_hh).
    const bool padded = p->mode != LSTM_MODE_LSTM;
    std::vector<const void *> wpad_ptrs;
    const void *const *wts = weights;
    int wper = per;
    bool bias_on = p->has_bias != 0;
    if (padded) {
        if (!sch.persistent || reserve) return LSTM_ERR_UNSUPPORTED;
        wpad_ptrs.assign((size_t)p->L * p->D * 4, nullptr);
        std::vector<PadJob> jobs;
        const int rows = p->NG * p->H;
        walk_padded_params(p, [&](int l, int d, int k, size_t off, size_t cols) {
            void *dst = ws + lay.wpad + off;
            wpad_ptrs[(size_t)(l * p->D + d) * 4 + k] = dst;
            const void *src = (k < 2 || p->has_bias) ? weights[(size_t)(l * p->D + d) * per + k] : nullptr;
            int valid = src ? rows : 0;
            if (k == 3 && p->mode == LSTM_MODE_GRU && src) valid = 2 * p->H;
            jobs.push_back(PadJob{src ? src : dst, dst, valid, 4 * p->H, (int)cols});
        });
        if (launch_pad_rows(jobs.data(), (int)jobs.size(), p->dtype, st) != hipSuccess) {
            (void)hipGetLastError();
            return LSTM_ERR_LAUNCH;
        }
        wts = wpad_ptrs.data();
        wper = 4;
        bias_on = true;
    }
    unsigned *status = reinterpret_cast<unsigned *>(ws + lay.status);
    unsigned long long *xbuf = reinterpret_cast<unsigned long long *>(ws + lay.xbuf);
    float *G = reinterpret_cast<float *>(ws + lay.G);
    float *cstate = reinterpret_cast<float *>(ws + lay.cstate);
    float *hstate = reinterpret_cast<float *>(ws + lay.hstate);
    int *dlen = lengths_h ? reinterpret_cast<int *>(ws + lay.lens) : nullptr;
    const size_t es = elem_size(p->dtype);
    const size_t state_elems = (size_t)p->D * B * p->H;
    if (dlen && hipMemcpyAsync(dlen, lengths_h, (size_t)B * sizeof(int), hipMemcpyHostToDevice, st) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_LAUNCH;
    }

    // per-step GEMM kernel: usable when the recurrence steps and every layer's
    // operands meet its alignment (checked before anything is enqueued)
    bool gemm = !sch.persistent && gemm_step_shape_ok(p);
    for (int l = 0; l < p->L && gemm; ++l) {
        RecArgs q{};
        for (int d = 0; d < p->D; ++d) q.whh[d] = weights[(size_t)(l * p->D + d) * per + 1];
        q.Y = l == p->L - 1 ? y : static_cast<void *>(ws + lay.ymid[l & 1]);
        q.h0 = h0 ? static_cast<const char *>(h0) + (size_t)l * state_elems * es : nullptr;
        q.H = p->H;
        q.D = p->D;
        q.T = T;
        q.bfirst = p->batch_first;
        gemm = rec_step_gemm_ok(q, p->dtype);
    }
    if (p->rec_mode == LSTM_REC_GEMM && !gemm) return LSTM_ERR_UNSUPPORTED;

    // Layer wavefront: every layer's recurrence (input products included) in
    // one cooperative launch.  If the runtime refuses that launch (nothing
    // ran), the layer-by-layer path below does the work.
    WaveSched wsch{};
    if (!padded && !dlen && !reserve && choose_wave(p, B, dev, &wsch)) {
        const size_t slot_words = (size_t)wsch.NGB * (size_t)((p->H + (p->dtype == LSTM_BF16 ? 31 : 15)) /
                                                              (p->dtype == LSTM_BF16 ? 32 : 16)) * 256;
        const size_t used_words = slot_words * ((size_t)T * (p->L - 1) + 2);
        uint32_t *xw = reinterpret_cast<uint32_t *>(ws + lay.G);  // the exchange slots live in G's place
        if (launch_fill_u32(status, kStatusBytes / sizeof(unsigned), 0u, st) != hipSuccess ||
            launch_fill_u32(xw, used_words, 0u, st) != hipSuccess)
            return LSTM_ERR_LAUNCH;
        WaveArgs qa{};
        size_t off_words = 0;
        for (int l = 0; l < p->L; ++l) {
            const void *const *w = weights + (size_t)l * per;
            qa.wih[l] = w[0];
            qa.whh[l] = w[1];
            qa.b_ih[l] = p->has_bias ? w[2] : nullptr;
            qa.b_hh[l] = p->has_bias ? w[3] : nullptr;
            qa.xbuf[l] = xw + off_words;
            off_words += slot_words * (l + 1 < p->L ? (size_t)T : 2);
        }
        qa.x = x;
        qa.h0 = h0;
        qa.c0 = c0;
        qa.Y = y;
        qa.hn = h_n;
        qa.cn = c_n;
        qa.status = status;
        qa.L = p->L;
        qa.T = T;
        qa.B = B;
        qa.H = p->H;
        qa.I = p->I;
        qa.P = wsch.P;
        qa.BG = wsch.BG;
        qa.NGB = wsch.NGB;
        qa.kch = (p->H + (p->dtype == LSTM_BF16 ? 31 : 15)) / (p->dtype == LSTM_BF16 ? 32 : 16);
        qa.ncx0 = wsch.ncx0;
        qa.map_xcd = wsch.map_xcd;
        qa.poll_sleep = p->poll_sleep;
        qa.pace = (int)((long long)(p->read_pace_ns >= 0 ? p->read_pace_ns : 375) * di.wall_khz / 1000000);
        const int per16w = p->dtype == LSTM_BF16 ? 8 : 4;
        // 16-byte fragment loads of W and h0 rows; x rows go through a buffer resource
        bool vec = (p->H % per16w == 0) && (p->I % per16w == 0) && (!h0 || (uintptr_t)h0 % 16 == 0) &&
                   (uintptr_t)x % 16 == 0;
        for (int l = 0; l < p->L; ++l)
            vec = vec && (uintptr_t)qa.whh[l] % 16 == 0 && (uintptr_t)qa.wih[l] % 16 == 0;
        qa.vec = vec ? 1 : 0;
        qa.timeout_ticks = (long long)di.wall_khz * 1000LL * 5;  // five seconds
        const int span = span_begin(p, st, 1);
        // x's fragment loads need 16-byte rows: otherwise the layer-by-layer path
        if (vec && (size_t)B * p->I * es < ((size_t)1 << 31) && launch_wave(qa, wsch.NT, p->dtype, wsch.lpw, st) == hipSuccess) {
            span_end(p, span, st, 1);
            if (p->timing) p->acc.calls += 1;
            return LSTM_OK;
        }
        (void)hipGetLastError();
        span_end(p, span, st, 0);
    }

    if (launch_fill_u32(status, lay.sync_bytes / sizeof(unsigned), 0u, st) != hipSuccess) return LSTM_ERR_LAUNCH;

    const int per16 = p->dtype == LSTM_BF16 ? 8 : 4;
    // small batches: each direction's recurrence on one XCD, after a hoisted projection
    const bool small = !padded && !dlen && !reserve && use_xcd(p, B, dev);
    // large batches whose layers would step: W_hh held once across the chip, h through y
    int res_groups = 0, res_slices = 0, res_map = 0;
    const bool res = !small && !padded && !dlen && !reserve &&
                     use_res(p, B, dev, sch.persistent, &res_groups, &res_slices, &res_map);
    // Exchange tags are one bit per word: bit p of xpar is the parity of the
    // writes exchange buffer p has received so far in this call.  A k_rec
    // layer writes buffer s & 1 at every step s < T - 1.
    unsigned xpar = 0;
    const unsigned layer_writes = (unsigned)((T / 2) & 1) | ((unsigned)(((T - 1) / 2) & 1) << 1);
    for (int l = 0; l < p->L; ++l) {
        // layer outputs below the top one: workspace ping-pong, or the
        // training reserve (the backward pass reads them again)
        auto mid = [&](int k) -> char * { return reserve ? reserve + rl.y(p, k) : ws + lay.ymid[k & 1]; };
        // training with dropout: a layer above the first reads the output below after dropout
        const bool drop = reserve && rl.dropout;
        const void *X = l == 0 ? x : drop ? static_cast<const void *>(reserve + rl.xd(p, l - 1))
                                          : static_cast<const void *>(mid(l - 1));
        void *Y = l == p->L - 1 ? y : static_cast<void *>(mid(l));
        const int in_l = l == 0 ? p->I : p->D * p->H;

        const void *wih[2] = {nullptr, nullptr};
        for (int d = 0; d < p->D; ++d) wih[d] = wts[(size_t)(l * p->D + d) * wper];
        // the GRU needs x W_in^T apart from W_hn h (reset product): never fused
        // (the resident recurrence reads G: the layer hoists its projection)
        const bool res_layer = res && res_ring_bytes(p->H, res_groups) <= lay.sync_bytes - lay.xbuf &&
                               (uintptr_t)Y % 16 == 0 &&
                               (!h0 || ((uintptr_t)h0 + (size_t)l * state_elems * es) % 16 == 0) &&
                               (uintptr_t)wts[(size_t)(l * p->D) * wper + 1] % 16 == 0 &&
                               (p->D < 2 || (uintptr_t)wts[(size_t)(l * p->D + 1) * wper + 1] % 16 == 0);
        int ncx = p->mode == LSTM_MODE_GRU || small || res_layer ? 0 : fused_chunks(p, sch, T, B, in_l, X, wih, di);

        // hoisted projection G = X W_ih^T + b_ih + b_hh (skipped when fused)
        auto project = [&]() -> bool {
            ProjArgs pa{};
            pa.X = X;
            pa.G = G;
            pa.M = T * B;
            pa.N = 4 * p->H;
            pa.K = in_l;
            pa.ldx = in_l;
            pa.D = p->D;
            for (int d = 0; d < p->D; ++d) {
                const void *const *w = wts + (size_t)(l * p->D + d) * wper;
                pa.W[d] = w[0];
                pa.b_ih[d] = bias_on ? w[2] : nullptr;
                pa.b_hh[d] = bias_on ? w[3] : nullptr;
            }
            const int sp = span_begin(p, st, 0);
            if (launch_proj(pa, p->dtype, p->proj_tile, st) != hipSuccess) {
                (void)hipGetLastError();
                return false;
            }
            span_end(p, sp, st, 1);
            return true;
        };
        if (ncx == 0 && !project()) return LSTM_ERR_LAUNCH;

        RecArgs ra{};
        for (int d = 0; d < p->D; ++d) {
            const void *const *w = wts + (size_t)(l * p->D + d) * wper;
            ra.whh[d] = w[1];
            ra.wih[d] = w[0];
            ra.b_ih[d] = bias_on ? w[2] : nullptr;
            ra.b_hh[d] = bias_on ? w[3] : nullptr;
            // the GRU's b_hn: from the caller's b_hh
            if (p->mode == LSTM_MODE_GRU)
                ra.b_hh[d] = p->has_bias ? weights[(size_t)(l * p->D + d) * per + 3] : nullptr;
        }
        ra.mode = p->mode;
        ra.ncx = ncx;
        ra.I = in_l;
        ra.x = X;
        ra.G = G;
        ra.h0 = h0 ? static_cast<const char *>(h0) + (size_t)l * state_elems * es : nullptr;
        ra.c0 = c0 ? c0 + (size_t)l * state_elems : nullptr;
        ra.Y = Y;
        ra.hn = h_n ? static_cast<char *>(h_n) + (size_t)l * state_elems * es : nullptr;
        ra.cn = c_n ? c_n + (size_t)l * state_elems : nullptr;
        ra.cstate = cstate;
        ra.hstate = hstate;
        ra.len = dlen;
        ra.bfirst = p->batch_first;
        ra.acts = reserve ? reinterpret_cast<float *>(reserve + rl.acts_layer * l) : nullptr;
        ra.xbuf = xbuf;
        ra.xpar = xpar;
        ra.xwide = sch.wide ? 1 : 0;
        ra.status = status;
        ra.T = T;
        ra.B = B;
        ra.H = p->H;
        ra.D = p->D;
        ra.P = sch.P;
        ra.BG = sch.BG;
        ra.NGB = sch.NGB;
        ra.kch = sch.geom.kch;
        ra.kchp = sch.geom.kchp;
        ra.nbatch = sch.geom.nbatch;
        ra.part_bufs = sch.geom.part_bufs;
        ra.poll_sleep = p->poll_sleep;
        ra.pace = (int)((long long)read_pace_for(p, sch) * di.wall_khz / 1000000);
        ra.map_xcd = sch.map_xcd;
        ra.wreg = sch.geom.wreg;
        ra.vec = (p->H % per16 == 0) && ((uintptr_t)Y % 16 == 0) && (!h0 || (uintptr_t)h0 % 16 == 0);
        for (int d = 0; d < p->D; ++d) ra.vec = ra.vec && ((uintptr_t)ra.whh[d] % 16 == 0);
        ra.timeout_ticks = (long long)di.wall_khz * 1000LL * 5;  // five seconds
        int span = span_begin(p, st, 1);
        if (small) {
            RecArgs xa = ra;
            xa.P = xcd_workgroups(p->H);
            // no default pace: on one XCD a stale read costs a short round trip
            xa.pace = (int)((long long)(p->read_pace_ns >= 0 ? p->read_pace_ns : 0) * di.wall_khz / 1000000);
            if (launch_xcd(xa, p->dtype, st) == hipSuccess) {
                span_end(p, span, st, 1);
                xpar ^= layer_writes;
                continue;
            }
            (void)hipGetLastError();  // refused (nothing ran): the general recurrence below
        }
        if (res_layer) {
            // The kernel's ring lives in the exchange buffer and starts zeroed
            // (tag 0).  The buffer is zeroed again after it, and the other
            // kernels' tag sequence restarts (xpar = 0): every word is then tag 0.
            RecArgs xa = ra;
            xa.NGB = res_groups;
            xa.P = res_slices;
            xa.map_xcd = res_map;
            unsigned *const xw = reinterpret_cast<unsigned *>(ws + lay.xbuf);
            const size_t xwords = (lay.sync_bytes - lay.xbuf) / sizeof(unsigned);
            if (launch_fill_u32(xw, xwords, 0u, st) != hipSuccess) {
                (void)hipGetLastError();
                return LSTM_ERR_LAUNCH;
            }
            const bool ran = launch_res(xa, st) == hipSuccess;
            if (!ran) (void)hipGetLastError();  // refused (nothing ran): the general recurrence below
            if (launch_fill_u32(xw, xwords, 0u, st) != hipSuccess) {
                (void)hipGetLastError();
                return LSTM_ERR_LAUNCH;
            }
            xpar = 0;
            if (ran) {
                span_end(p, span, st, 1);
                continue;
            }
        }
        bool stepped = !sch.persistent;
        if (sch.persistent) {
            ra.s_begin = 0;
            ra.s_end = T;
            hipError_t e = launch_rec(ra, sch.tile, sch.smem, p->dtype, true, st);
            if (e != hipSuccess && ra.ncx > 0) {
                // the fused launch was refused (nothing ran): hoist the
                // projection and try the plain kernel
                (void)hipGetLastError();
                span_end(p, span, st, 0);
                ra.ncx = 0;
                if (!project()) return LSTM_ERR_LAUNCH;
                span = span_begin(p, st, 1);
                e = launch_rec(ra, sch.tile, sch.smem, p->dtype, true, st);
            }
            if (e != hipSuccess) {
                (void)hipGetLastError();
                // The cooperative launch was refused (nothing ran): in automatic
                // mode the layer falls back to one launch per step.
                if (p->rec_mode == LSTM_REC_PERSISTENT) return LSTM_ERR_LAUNCH;
                stepped = true;
            }
        }
        bool use_gemm_layer = false;
        if (stepped) {
            // (k_rec_step's LSTM instance needs real LSTM parameters: not for the padded modes)
            const bool use_gemm = !padded && (gemm || (sch.persistent && gemm_step_shape_ok(p) &&
                                                       rec_step_gemm_ok(ra, p->dtype)));
            use_gemm_layer = use_gemm;
            for (int s = 0; s < T; ++s) {
                ra.s_begin = s;
                ra.s_end = s + 1;
                const hipError_t e = use_gemm ? launch_rec_step_gemm(ra, p->dtype, st)
                                              : launch_rec(ra, sch.tile, sch.smem, p->dtype, false, st);
                if (e != hipSuccess) {
                    (void)hipGetLastError();
                    return LSTM_ERR_LAUNCH;
                }
            }
        }
        span_end(p, span, st, stepped ? T : 1);
        if (!use_gemm_layer) xpar ^= layer_writes;  // k_rec_step writes no exchange words
        // k_rec_step leaves the unchanged h in y at padded steps (the next step
        // reads it there); the caller sees zeros
        if (dlen && use_gemm_layer && l == p->L - 1 &&
            launch_mask_padded(y, dlen, T, B, (size_t)p->D * p->H * es, p->batch_first != 0, st) != hipSuccess)
            return LSTM_ERR_LAUNCH;
        if (drop && l + 1 < p->L) {
            const double q = p->dropout;
            const unsigned long long thr = q >= 1.0 ? (1ull << 53) : (unsigned long long)std::ceil(q * 0x1p53);
            const float scale = q >= 1.0 ? 0.f : (float)(1.0 / (1.0 - q));
            if (launch_dropout_fwd(Y, reserve + rl.xd(p, l), reinterpret_cast<unsigned char *>(reserve + rl.keep(p, l)),
                                   T, B, p->D * p->H, p->drop_seed, p->drop_call, l, thr, scale, p->dtype,
                                   p->batch_first != 0, st) != hipSuccess) {
                (void)hipGetLastError();
                return LSTM_ERR_LAUNCH;
            }
        }
    }
    if (p->timing) p->acc.calls += 1;
    return LSTM_OK;
}

// The GRU and the RNNs take the persistent recurrence when its schedule
// applies (unless the caller asked for stepping) and the per-step GEMM kernel
// otherwise.
bool use_persistent_for_mode(const lstm_plan *p, int B, bool wide) {
    if (p->rec_mode == LSTM_REC_STEP || p->rec_mode == LSTM_REC_GEMM || B < 1) return false;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    Sched s{};
    return choose_sched(p, B, dev, &s, wide) == LSTM_OK && s.persistent;
}

// The forward pass of the GRU and the plain RNNs: per layer the hoisted
// projection G = X W_ih^T + b_ih (both directions), then one k_rec_step launch
// per step, which adds W_hh h_{t-1} + b_hh and applies the mode's update.
lstm_status forward_modes(lstm_plan *p, const void *x, const int *lengths_h, const void *h0,
                          const void *const *weights, int T, int B, int layers, int bidir, void *y, void *h_n,
                          const float *c_n, void *workspace, size_t workspace_bytes, void *stream_,
                          bool own_ws = false) {
    Layout lay;
    int rc = validate(p, x, h0, nullptr, weights, T, B, layers, bidir, y, workspace, workspace_bytes, &lay);
    if (rc != LSTM_OK) return (lstm_status)rc;
    if (c_n) return LSTM_ERR_ARG;  // no cell state
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    const int per = p->has_bias ? 4 : 2;
    const void *ptrs[] = {x, y, own_ws ? nullptr : workspace, h0, h_n};
    for (const void *q : ptrs)
        if (q && !is_device_ptr(q, dev)) return LSTM_ERR_DEVICE;
    for (int i = 0; i < p->L * p->D * per; ++i)
        if (!is_device_ptr(weights[i], dev)) return LSTM_ERR_DEVICE;
    hipStream_t st = static_cast<hipStream_t>(stream_);
    char *ws = static_cast<char *>(workspace);
    float *G = reinterpret_cast<float *>(ws + lay.G);
    const size_t es = elem_size(p->dtype), state_elems = (size_t)p->D * B * p->H;
    int *dlen = lengths_h ? reinterpret_cast<int *>(ws + lay.lens) : nullptr;
    auto layer_args = [&](int l) {
        RecArgs ra{};
        for (int d = 0; d < p->D; ++d) {
            const void *const *w = weights + (size_t)(l * p->D + d) * per;
            ra.whh[d] = w[1];
            ra.b_hh[d] = p->has_bias ? w[3] : nullptr;
        }
        ra.G = G;
        ra.h0 = h0 ? static_cast<const char *>(h0) + (size_t)l * state_elems * es : nullptr;
        ra.Y = l == p->L - 1 ? y : static_cast<void *>(ws + lay.ymid[l & 1]);
        ra.hn = h_n ? static_cast<char *>(h_n) + (size_t)l * state_elems * es : nullptr;
        ra.T = T;
        ra.B = B;
        ra.H = p->H;
        ra.D = p->D;
        ra.bfirst = p->batch_first;
        ra.mode = p->mode;
        ra.len = dlen;
        return ra;
    };
    // every layer's operands must suit the per-step kernel: checked before anything is enqueued
    for (int l = 0; l < p->L; ++l)
        if (!rec_step_gemm_ok(layer_args(l), p->dtype)) return LSTM_ERR_UNSUPPORTED;
    if (dlen && hipMemcpyAsync(dlen, lengths_h, (size_t)B * sizeof(int), hipMemcpyHostToDevice, st) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_LAUNCH;
    }
    for (int l = 0; l < p->L; ++l) {
        const void *X = l == 0 ? x : static_cast<const void *>(ws + lay.ymid[(l - 1) & 1]);
        const int in_l = l == 0 ? p->I : p->D * p->H;
        ProjArgs pa{};
        pa.X = X;
        pa.G = G;
        pa.M = T * B;
        pa.N = p->NG * p->H;
        pa.K = in_l;
        pa.ldx = in_l;
        pa.D = p->D;
        for (int d = 0; d < p->D; ++d) {
            const void *const *w = weights + (size_t)(l * p->D + d) * per;
            pa.W[d] = w[0];
            pa.b_ih[d] = p->has_bias ? w[2] : nullptr;  // b_hh joins in the step
        }
        int span = span_begin(p, st, 0);
        if (launch_proj(pa, p->dtype, p->proj_tile, st) != hipSuccess) {
            (void)hipGetLastError();
            return LSTM_ERR_LAUNCH;
        }
        span_end(p, span, st, 1);
        RecArgs ra = layer_args(l);
        span = span_begin(p, st, 1);
        for (int s = 0; s < T; ++s) {
            ra.s_begin = s;
            ra.s_end = s + 1;
            if (launch_rec_step_gemm(ra, p->dtype, st) != hipSuccess) {
                (void)hipGetLastError();
                return LSTM_ERR_LAUNCH;
            }
        }
        span_end(p, span, st, T);
    }
    // padded steps carried h in y for the next step; the caller sees zeros
    if (dlen && launch_mask_padded(y, dlen, T, B, (size_t)p->D * p->H * es, p->batch_first != 0, st) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_LAUNCH;
    }
    if (p->timing) p->acc.calls += 1;
    return LSTM_OK;
}

}  // namespace

lstm_status lstm_amd::forward_dispatch(lstm_plan *p, const void *x, const void *h0, const float *c0,
                                       const void *const *weights, int T, int B, int layers, int bidir, void *y,
                                       void *h_n, float *c_n, void *workspace, size_t workspace_bytes,
                                       void *stream, bool own_ws) {
    if (p && p->mode != LSTM_MODE_LSTM) {
        if (c0 || c_n) return LSTM_ERR_ARG;  // no cell state
        // the persistent kernel on padded gate slots where the schedule allows, else one launch per step
        if (use_persistent_for_mode(p, B, needs_wide_exchange(p, h0 != nullptr, false)))
            return forward_impl(p, x, nullptr, h0, nullptr, weights, T, B, layers, bidir, y, h_n, nullptr,
                                workspace, workspace_bytes, stream, nullptr, own_ws);
        return forward_modes(p, x, nullptr, h0, weights, T, B, layers, bidir, y, h_n, c_n, workspace,
                             workspace_bytes, stream, own_ws);
    }
    return forward_impl(p, x, nullptr, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, workspace,
                        workspace_bytes, stream, nullptr, own_ws);
}

extern "C" {

lstm_status lstm_forward(lstm_plan *p, const void *x, const void *h0, const float *c0,
                         const void *const *weights, int T, int B, int layers, int bidir, void *y,
                         void *h_n, float *c_n, void *workspace, size_t workspace_bytes, void *stream) {
    return forward_dispatch(p, x, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, workspace, workspace_bytes,
                            stream, false);
}

lstm_status lstm_reserve_size(const lstm_plan *p, int T, int B, size_t *bytes) {
    if (!p || !bytes) return LSTM_ERR_ARG;
    if (p->mode != LSTM_MODE_LSTM) return LSTM_ERR_UNSUPPORTED;
    ReserveLayout rl{};
    if (!make_reserve(p, T, B, &rl)) return LSTM_ERR_SHAPE;
    *bytes = rl.total;
    return LSTM_OK;
}

static lstm_status forward_train_impl(lstm_plan *p, const void *x, const int *lengths, const void *h0,
                                      const float *c0, const void *const *weights, int T, int B, int layers,
                                      int bidir, void *y, void *h_n, float *c_n, void *reserve, size_t reserve_bytes,
                                      void *workspace, size_t workspace_bytes, void *stream) {
    if (!p || !reserve) return LSTM_ERR_ARG;
    if (lengths) {
        if (T < 1 || B < 1) return LSTM_ERR_SHAPE;
        for (int b = 0; b < B; ++b)
            if (lengths[b] < 1 || lengths[b] > T) return LSTM_ERR_ARG;
    }
    if (p->mode != LSTM_MODE_LSTM) return LSTM_ERR_UNSUPPORTED;
    ReserveLayout rl{};
    if (!make_reserve(p, T, B, &rl)) return LSTM_ERR_SHAPE;
    if (reserve_bytes < rl.total) return LSTM_ERR_WORKSPACE;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    if (!is_device_ptr(reserve, dev)) return LSTM_ERR_DEVICE;
    const lstm_status s = forward_impl(p, x, lengths, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, workspace,
                                       workspace_bytes, stream, static_cast<char *>(reserve));
    if (s == LSTM_OK && rl.dropout) p->drop_call += 1;  // the next call draws a fresh mask
    return s;
}

lstm_status lstm_forward_train(lstm_plan *p, const void *x, const void *h0, const float *c0,
                               const void *const *weights, int T, int B, int layers, int bidir, void *y,
                               void *h_n, float *c_n, void *reserve, size_t reserve_bytes, void *workspace,
                               size_t workspace_bytes, void *stream) {
    return forward_train_impl(p, x, nullptr, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, reserve,
                              reserve_bytes, workspace, workspace_bytes, stream);
}

lstm_status lstm_forward_train_lengths(lstm_plan *p, const void *x, const int *lengths, const void *h0,
                                       const float *c0, const void *const *weights, int T, int B, int layers,
                                       int bidir, void *y, void *h_n, float *c_n, void *reserve, size_t reserve_bytes,
                                       void *workspace, size_t workspace_bytes, void *stream) {
    if (!lengths) return LSTM_ERR_ARG;
    return forward_train_impl(p, x, lengths, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, reserve,
                              reserve_bytes, workspace, workspace_bytes, stream);
}

lstm_status lstm_backward_workspace_size(const lstm_plan *p, int T, int B, size_t *bytes) {
    if (!p || !bytes) return LSTM_ERR_ARG;
    if (p->mode != LSTM_MODE_LSTM) return LSTM_ERR_UNSUPPORTED;
    BwdLayout bl{};
    if (!make_bwd_layout(p, T, B, &bl)) return LSTM_ERR_SHAPE;
    *bytes = bl.total;
    return LSTM_OK;
}

// lengths_h: NULL (every row has T steps) or B host values, validated here
static lstm_status backward_impl(lstm_plan *p, const void *x, const int *lengths_h, const void *h0, const float *c0,
                                 const void *const *weights, const void *y, const void *dy, const void *dh_n,
                                 const float *dc_n, const void *reserve, size_t reserve_bytes, int T, int B,
                                 int layers, int bidir, void *dx, void *dh0, float *dc0, void *const *dweights,
                                 void *workspace, size_t workspace_bytes, void *stream_) {
    if (!p || !x || !weights || !y || !dy || !reserve || !dweights || !workspace) return LSTM_ERR_ARG;
    if (layers != p->L || (bidir != 0) != (p->D == 2) || T < 1 || B < 1) return LSTM_ERR_SHAPE;
    if (lengths_h)
        for (int b = 0; b < B; ++b)
            if (lengths_h[b] < 1 || lengths_h[b] > T) return LSTM_ERR_ARG;
    if ((h0 == nullptr) != (c0 == nullptr)) return LSTM_ERR_ARG;
    if (p->mode != LSTM_MODE_LSTM) return LSTM_ERR_UNSUPPORTED;
    const int per = p->has_bias ? 4 : 2;
    for (int i = 0; i < p->L * p->D * per; ++i)
        if (!weights[i] || !dweights[i]) return LSTM_ERR_ARG;
    ReserveLayout rl{};
    BwdLayout bl{};
    if (!make_reserve(p, T, B, &rl) || !make_bwd_layout(p, T, B, &bl)) return LSTM_ERR_SHAPE;
    if (reserve_bytes < rl.total || workspace_bytes < bl.total) return LSTM_ERR_WORKSPACE;
    // the backward cell reads one step's activations ([B, D, 5H] floats) and
    // the [D, B, H] state arrays with 32-bit byte offsets
    if ((size_t)B * p->D * 5 * p->H * sizeof(float) >= ((size_t)1 << 31)) return LSTM_ERR_UNSUPPORTED;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    const void *ptrs[] = {x, h0, c0, y, dy, dh_n, dc_n, reserve, dx, dh0, dc0, workspace};
    for (const void *q : ptrs)
        if (q && !is_device_ptr(q, dev)) return LSTM_ERR_DEVICE;
    for (int i = 0; i < p->L * p->D * per; ++i)
        if (!is_device_ptr(weights[i], dev) || !is_device_ptr(dweights[i], dev)) return LSTM_ERR_DEVICE;

    hipStream_t st = static_cast<hipStream_t>(stream_);
    char *ws = static_cast<char *>(workspace);
    const char *res = static_cast<const char *>(reserve);
    char *dz = ws + bl.dz;
    // dz and the operands of every backward product, in the gradient dtype
    // gdt: bf16 for bf16 parameters with an even H (fp32 accumulation, the
    // cell math and the carries stay fp32, results rounded once), else fp32
    const int gdt = p->dtype == LSTM_BF16 && p->H % 2 == 0 ? DT_BF16 : DT_F32;
    const size_t ges = gdt == DT_BF16 ? 2 : 4;
    char *dzt = ws + bl.dzt;   // one direction's dz^T
    char *xt = ws + bl.xt;
    char *ht = ws + bl.ht;
    float *dyb[2] = {reinterpret_cast<float *>(ws + bl.dy[0]), reinterpret_cast<float *>(ws + bl.dy[1])};
    float *dcb = reinterpret_cast<float *>(ws + bl.dc);
    float *dhnb = reinterpret_cast<float *>(ws + bl.dhn);
    char *wht = ws + bl.wht;
    char *wcat = ws + bl.wcat;
    float *ksp = reinterpret_cast<float *>(ws + bl.ksp);
    float *db = reinterpret_cast<float *>(ws + bl.db);
    const int dt = p->dtype, H = p->H, D = p->D, G4 = 4 * H;
    const size_t es = elem_size(p->dtype), TB = (size_t)T * B, BH = (size_t)B * H, DBH = (size_t)D * BH;
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    auto fail = []() {
        (void)hipGetLastError();
        return LSTM_ERR_LAUNCH;
    };
    // out[M][N] = A[M][K] Bm[N][K]^T in fp32, rounded once to out_dt; split
    // over K (slabs in ksp, summed in order) when the product has few output
    // tiles, else computed into f32 (out itself when out_dt is fp32)
    auto gemm_nt = [&](const void *A, int lda, const void *Bm, int M, int N, int K, void *out, int out_dt,
                       float *f32) {
        ProjArgs g{};
        g.X = A;
        g.W[0] = Bm;
        g.M = M;
        g.N = N;
        g.K = K;
        g.ldx = lda;
        g.D = 1;
        g.kchunk = proj_kchunk(M, N, K);
        const size_t mn = (size_t)M * N;
        const int sp = span_begin(p, st, 3);
        struct End {
            lstm_plan *p;
            int sp;
            hipStream_t st;
            ~End() { span_end(p, sp, st, 1); }
        } end{p, sp, st};
        if (g.kchunk) {
            g.G = ksp;
            return ok(launch_proj(g, gdt, 0, st)) &&
                   ok(launch_ksum(ksp, (K + g.kchunk - 1) / g.kchunk, mn, mn, out, out_dt, st));
        }
        if (out_dt == DT_F32) {
            g.G = static_cast<float *>(out);
            return ok(launch_proj(g, gdt, 0, st));
        }
        g.G = f32;
        return ok(launch_proj(g, gdt, 0, st)) && ok(launch_cast_to(f32, out, mn, out_dt, st));
    };
    if (p->timing) p->acc.bwd_calls += 1;
    // per-row lengths on the device, and the gradient of h carried through padded steps
    int *dlen = lengths_h ? reinterpret_cast<int *>(ws + bl.lens) : nullptr;
    if (dlen && hipMemcpyAsync(dlen, lengths_h, (size_t)B * sizeof(int), hipMemcpyHostToDevice, st) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_LAUNCH;
    }
    // The recurrent product of a backward step: a 16x16 tile per workgroup
    // over the whole K = 4H, or, when those tiles leave CUs idle, its K split
    // between two workgroups (all resident at once: at most one per CU).
    // The status word and the hand-over buffer start at zero in every call,
    // and each step launch gets a tag of its own.
    const DevInfo di = dev_info(dev);
    const long long tiles = (long long)((B + 15) / 16) * ((H + 15) / 16) * D;
    const int ksplit = di.ok && 2 * tiles <= di.cus ? 2 : 1;
    unsigned *bstatus = reinterpret_cast<unsigned *>(ws + bl.status);
    auto *pbuf = reinterpret_cast<unsigned long long *>(ws + bl.pbuf);
    const long long timeout_ticks = (long long)(di.ok ? di.wall_khz : 100000) * 1000LL * 2;  // two seconds
    unsigned step_tag = 0;
    if (launch_fill_u32(bstatus, (bl.dz - bl.status) / sizeof(unsigned), 0u, st) != hipSuccess) return LSTM_ERR_LAUNCH;
    // the gradient of the top layer's output, as fp32
    int cur = 0;
    // batch-first x, y, dy, dx: the internal gradient buffers stay time-major
    const bool bfirst = p->batch_first != 0;
    if (!ok(bfirst ? launch_permute_rows(dy, dyb[cur], T, B, D * H, dt, DT_F32, true, st)
                   : launch_cast_from(dy, dyb[cur], TB * D * H, dt, st)))
        return fail();
    for (int l = p->L - 1; l >= 0; --l) {
        const int in_l = l == 0 ? p->I : D * H;
        const void *X = l == 0 ? x : static_cast<const void *>(res + (rl.dropout ? rl.xd(p, l - 1) : rl.y(p, l - 1)));
        const void *Y = l == p->L - 1 ? y : static_cast<const void *>(res + rl.y(p, l));
        const float *acts = reinterpret_cast<const float *>(res + rl.acts_layer * l);
        const float *c0l = c0 ? c0 + (size_t)l * DBH : nullptr;
        const char *h0l = h0 ? static_cast<const char *>(h0) + (size_t)l * DBH * es : nullptr;
        // W_hh^T per direction for the recurrent products
        for (int d = 0; d < D; ++d)
            if (!ok(launch_transpose(weights[(size_t)(l * D + d) * per + 1], H, G4, H, wht + (size_t)d * H * G4 * ges,
                                     G4, dt, gdt, st)))
                return fail();
        if (dh_n && !ok(launch_cast_from(static_cast<const char *>(dh_n) + (size_t)l * DBH * es, dhnb, DBH, dt, st)))
            return fail();
        const int rec_span = span_begin(p, st, 2);
        // the recurrence, backwards: sb = 0 is each direction's last step;
        // launch sb multiplies step sb's dz by W_hh and runs step sb + 1's cell
        BwdCellArgs ca{};
        ca.acts = acts;
        ca.c0 = c0l;
        ca.dY = dyb[cur];
        ca.dhn = dh_n ? dhnb : nullptr;
        ca.dcn = dc_n ? dc_n + (size_t)l * DBH : nullptr;
        ca.dz = dz;
        ca.dc = dcb;
        ca.len = dlen;
        ca.dhc = reinterpret_cast<float *>(ws + bl.dhc);
        ca.T = T;
        ca.B = B;
        ca.H = H;
        ca.D = D;
        if (!ok(launch_bwd_cell(ca, gdt, st))) return fail();
        void *dh0l = dh0 ? static_cast<char *>(dh0) + (size_t)l * DBH * es : nullptr;
        for (int sb = 0; sb < T; ++sb) {
            BwdMmArgs ma{};
            ma.dz = dz;
            ma.whT = wht;
            ma.T = T;
            ma.B = B;
            ma.H = H;
            ma.D = D;
            ma.sb = sb;
            ma.ksplit = ksplit;
            ma.tag = ++step_tag;
            ma.pbuf = pbuf;
            ma.status = bstatus;
            ma.timeout_ticks = timeout_ticks;
            if (!ok(launch_bwd_step(ma, ca, dh0l, gdt, dt, st))) return fail();
        }
        span_end(p, rec_span, st, T);
        if (dc0 && hipMemcpyAsync(dc0 + (size_t)l * DBH, dcb, DBH * sizeof(float), hipMemcpyDeviceToDevice, st) !=
                       hipSuccess)
            return fail();
        // weight gradients: dW_ih = dz^T x, dW_hh = dz^T h_prev (operands in
        // gdt), db = sum of dz (fp32 column sums in fixed chunks, then in order)
        if (!ok(launch_transpose(X, in_l, (int)TB, in_l, xt, TB, dt, gdt, st, bfirst ? T : 0, B))) return fail();
        for (int d = 0; d < D; ++d) {
            void *const *dwd = dweights + (size_t)(l * D + d) * per;
            if (!ok(launch_transpose(dz + (size_t)d * G4 * ges, (size_t)D * G4, (int)TB, G4, dzt, TB, gdt, gdt, st)) ||
                !ok(launch_hprev_t(Y, (size_t)D * H, h0l ? h0l + (size_t)d * BH * es : nullptr, dlen, T, B, H, d, ht, dt,
                                   gdt, st, bfirst)))
                return fail();
            if (!gemm_nt(dzt, (int)TB, xt, G4, in_l, (int)TB, dwd[0], dt, ksp) ||
                !gemm_nt(dzt, (int)TB, ht, G4, H, (int)TB, dwd[1], dt, ksp))
                return fail();
            if (p->has_bias) {
                const int chunk = (int)((TB + kBiasChunks - 1) / kBiasChunks);
                const int nch = (int)((TB + chunk - 1) / chunk);
                if (!ok(launch_colsum_part(dz + (size_t)d * G4 * ges, (size_t)D * G4, (int)TB, G4, kBiasChunks, db, gdt,
                                           st)) ||
                    !ok(launch_ksum(db, nch, G4, G4, dwd[2], dt, st)) || !ok(launch_ksum(db, nch, G4, G4, dwd[3], dt, st)))
                    return fail();
            }
        }
        // input gradient dX = sum over directions of dz W_ih, the next dY
        if (l > 0 || dx) {
            for (int d = 0; d < D; ++d)
                if (!ok(launch_transpose(weights[(size_t)(l * D + d) * per], in_l, G4, in_l,
                                         wcat + (size_t)d * G4 * ges, (size_t)D * G4, dt, gdt, st)))
                    return fail();
            const bool out_dx = l == 0;
            if (out_dx && bfirst) {  // time-major rows in fp32, then into dx's batch-first rows
                if (!gemm_nt(dz, D * G4, wcat, (int)TB, in_l, D * G4, dyb[cur ^ 1], DT_F32, dyb[cur ^ 1]) ||
                    !ok(launch_permute_rows(dyb[cur ^ 1], dx, T, B, in_l, DT_F32, dt, false, st)))
                    return fail();
            } else if (!gemm_nt(dz, D * G4, wcat, (int)TB, in_l, D * G4, out_dx ? dx : dyb[cur ^ 1],
                                out_dx ? dt : DT_F32, dyb[cur ^ 1])) {
                return fail();
            }
            // through the dropout the layer below's output was sent up with
            if (!out_dx && rl.dropout) {
                const float scale = p->dropout >= 1.0 ? 0.f : (float)(1.0 / (1.0 - p->dropout));
                if (!ok(launch_dropout_bwd(dyb[cur ^ 1], reinterpret_cast<const unsigned char *>(res + rl.keep(p, l - 1)),
                                           TB * in_l, scale, st)))
                    return fail();
            }
        }
        cur ^= 1;
    }
    return LSTM_OK;
}

lstm_status lstm_backward(lstm_plan *p, const void *x, const void *h0, const float *c0,
                          const void *const *weights, const void *y, const void *dy, const void *dh_n,
                          const float *dc_n, const void *reserve, size_t reserve_bytes, int T, int B, int layers,
                          int bidir, void *dx, void *dh0, float *dc0, void *const *dweights, void *workspace,
                          size_t workspace_bytes, void *stream) {
    return backward_impl(p, x, nullptr, h0, c0, weights, y, dy, dh_n, dc_n, reserve, reserve_bytes, T, B, layers,
                         bidir, dx, dh0, dc0, dweights, workspace, workspace_bytes, stream);
}

lstm_status lstm_backward_lengths(lstm_plan *p, const void *x, const int *lengths, const void *h0, const float *c0,
                                  const void *const *weights, const void *y, const void *dy, const void *dh_n,
                                  const float *dc_n, const void *reserve, size_t reserve_bytes, int T, int B,
                                  int layers, int bidir, void *dx, void *dh0, float *dc0, void *const *dweights,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    if (!lengths) return LSTM_ERR_ARG;
    return backward_impl(p, x, lengths, h0, c0, weights, y, dy, dh_n, dc_n, reserve, reserve_bytes, T, B, layers,
                         bidir, dx, dh0, dc0, dweights, workspace, workspace_bytes, stream);
}

lstm_status lstm_forward_lengths(lstm_plan *p, const void *x, const int *lengths, const void *h0,
                                 const float *c0, const void *const *weights, int T, int B, int layers,
                                 int bidir, void *y, void *h_n, float *c_n, void *workspace,
                                 size_t workspace_bytes, void *stream) {
    if (!lengths) return LSTM_ERR_ARG;
    if (T < 1 || B < 1) return LSTM_ERR_SHAPE;
    for (int b = 0; b < B; ++b)
        if (lengths[b] < 1 || lengths[b] > T) return LSTM_ERR_ARG;
    if (p && p->mode != LSTM_MODE_LSTM) {
        if (c0 || c_n) return LSTM_ERR_ARG;  // no cell state
        if (use_persistent_for_mode(p, B, needs_wide_exchange(p, h0 != nullptr, true)))
            return forward_impl(p, x, lengths, h0, nullptr, weights, T, B, layers, bidir, y, h_n, nullptr,
                                workspace, workspace_bytes, stream);
        return forward_modes(p, x, lengths, h0, weights, T, B, layers, bidir, y, h_n, c_n, workspace,
                             workspace_bytes, stream);
    }
    return forward_impl(p, x, lengths, h0, c0, weights, T, B, layers, bidir, y, h_n, c_n, workspace,
                        workspace_bytes, stream);
}

// Packed sequences: the padded buffers and the row map after the forward's
// own workspace.  batch_sizes as documented in lstm.h.
struct PackLayout {
    size_t fwd, xpad, ypad, map, total;
    int B;
    size_t N;
};

static lstm_status pack_layout(const lstm_plan *p, const int *batch_sizes, int T, PackLayout *o) {
    if (!p || !batch_sizes) return LSTM_ERR_ARG;
    if (T < 1) return LSTM_ERR_SHAPE;
    if (batch_sizes[0] < 1) return LSTM_ERR_ARG;
    size_t n = 0;
    for (int t = 0; t < T; ++t) {
        if (batch_sizes[t] < 1 || (t > 0 && batch_sizes[t] > batch_sizes[t - 1])) return LSTM_ERR_ARG;
        n += (size_t)batch_sizes[t];
    }
    if (n > (size_t)INT_MAX) return LSTM_ERR_SHAPE;
    o->B = batch_sizes[0];
    o->N = n;
    size_t fwd = 0;
    const lstm_status rc = lstm_workspace_size(p, T, o->B, &fwd);
    if (rc != LSTM_OK) return rc;
    const size_t es = elem_size(p->dtype), rows = (size_t)T * o->B;
    size_t xb, yb;
    if (!mul_ok(rows, (size_t)p->I * es, &xb) || !mul_ok(rows, (size_t)p->D * p->H * es, &yb)) return LSTM_ERR_SHAPE;
    o->fwd = fwd;
    o->xpad = align_up(fwd);
    o->ypad = o->xpad + align_up(xb);
    o->map = o->ypad + align_up(yb);
    o->total = o->map + align_up(n * sizeof(int));
    return LSTM_OK;
}

lstm_status lstm_packed_workspace_size(const lstm_plan *p, const int *batch_sizes, int T, size_t *bytes) {
    if (!bytes) return LSTM_ERR_ARG;
    PackLayout pl{};
    const lstm_status rc = pack_layout(p, batch_sizes, T, &pl);
    if (rc != LSTM_OK) return rc;
    *bytes = pl.total;
    return LSTM_OK;
}

lstm_status lstm_forward_packed(lstm_plan *p, const void *x, const int *batch_sizes, int T, const void *h0,
                                const float *c0, const void *const *weights, int layers, int bidir, void *y,
                                void *h_n, float *c_n, void *workspace, size_t workspace_bytes, void *stream) {
    PackLayout pl{};
    lstm_status rc = pack_layout(p, batch_sizes, T, &pl);
    if (rc != LSTM_OK) return rc;
    if (!x || !y || !workspace) return LSTM_ERR_ARG;
    if (p->batch_first) return LSTM_ERR_UNSUPPORTED;  // the packed layout is time-major
    if (workspace_bytes < pl.total) return LSTM_ERR_WORKSPACE;
    const int B = pl.B;
    // row length of each sequence, and the padded row (t*B + b) of every packed row
    std::vector<int> lengths((size_t)B, 0), map(pl.N);
    size_t r = 0;
    for (int t = 0; t < T; ++t)
        for (int b = 0; b < batch_sizes[t]; ++b) {
            lengths[(size_t)b] = t + 1;
            map[r++] = t * B + b;
        }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    if (!is_device_ptr(x, dev) || !is_device_ptr(y, dev) || !is_device_ptr(workspace, dev)) return LSTM_ERR_DEVICE;
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    int *dmap = reinterpret_cast<int *>(ws + pl.map);
    const size_t es = elem_size(p->dtype);
    const size_t xrow = (size_t)p->I * es, yrow = (size_t)p->D * p->H * es;
    const size_t xwords = (pl.ypad - pl.xpad) / sizeof(unsigned);  // the padded x region, 256-byte aligned
    if (hipMemcpyAsync(dmap, map.data(), pl.N * sizeof(int), hipMemcpyHostToDevice, st) != hipSuccess ||
        launch_fill_u32(reinterpret_cast<unsigned *>(ws + pl.xpad), xwords, 0u, st) != hipSuccess ||
        launch_copy_rows(x, ws + pl.xpad, dmap, (int)pl.N, xrow, true, st) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_LAUNCH;
    }
    rc = lstm_forward_lengths(p, ws + pl.xpad, lengths.data(), h0, c0, weights, T, B, layers, bidir, ws + pl.ypad,
                              h_n, c_n, workspace, pl.fwd, stream);
    if (rc != LSTM_OK) return rc;
    if (launch_copy_rows(ws + pl.ypad, y, dmap, (int)pl.N, yrow, false, st) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_LAUNCH;
    }
    return LSTM_OK;
}

lstm_status lstm_device_status(const void *workspace, size_t workspace_bytes, void *stream,
                               unsigned *device_flags) {
    if (!workspace || !device_flags || workspace_bytes < kStatusBytes) return LSTM_ERR_ARG;
    hipStream_t st = static_cast<hipStream_t>(stream);
    unsigned v = 0;
    if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess) {
        (void)hipGetLastError();
        return LSTM_ERR_DEVICE;
    }
    *device_flags = v;
    return v ? LSTM_ERR_DEVICE_TIMEOUT : LSTM_OK;
}

}  // extern "C"
