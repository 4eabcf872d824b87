// Engine and C ABI of libgpt2.so: configuration checks, the arena layout, and the launch
// sequences of one GPT-2 training step (forward + loss, backward, AdamW) on one HIP stream.
//
// The model is GPT-2's pre-LN decoder ("Criei GPT-2 do zero com uma RTX 4090", sections "Ambiente"
// and "Configuração do treinamento": GPT-2 small built the nanoGPT way, vocabulary padded to a
// multiple of 128) trained on next-token cross-entropy with AdamW ("Pré-treinar um LLM: dados,
// compute, leis de escala e custo", opening paragraph). Everything below only sequences kernels;
// all arithmetic of the step runs in the .hip kernel files.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/gpt2.h"
#include "common.h"
#include "kernels.h"

namespace {

thread_local std::string g_err = "no error";

gpt2_status fail(gpt2_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define HIPCHK(x)                                                                  \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess)                                                          \
      return fail(GPT2_E_HIP, std::string(#x) + " failed: " + hipGetErrorString(e_)); \
  } while (0)

constexpr int LN_ROWS_PER_BLOCK = 16;
constexpr int COLSUM_ROWS_PER_BLOCK = 16;
constexpr int MAX_ROWS = 65536;
constexpr int TIMING_CAP = 4096;

// ------------------------------------------------------------------------------ geometry
struct Geo {
  int L, d, H, hd, T, B, M, V, Vp;
  bool bf16;
  int64_t N, P_layer;
  int64_t wte, wpe, layer0, lnfg, lnfb;
  int64_t lay(int l) const { return layer0 + (int64_t)l * P_layer; }
  int64_t ln1g(int l) const { return lay(l); }
  int64_t ln1b(int l) const { return lay(l) + d; }
  int64_t wqkv(int l) const { return lay(l) + 2 * (int64_t)d; }
  int64_t bqkv(int l) const { return wqkv(l) + 3 * (int64_t)d * d; }
  int64_t wo(int l) const { return bqkv(l) + 3 * (int64_t)d; }
  int64_t bo(int l) const { return wo(l) + (int64_t)d * d; }
  int64_t ln2g(int l) const { return bo(l) + d; }
  int64_t ln2b(int l) const { return ln2g(l) + d; }
  int64_t wfc(int l) const { return ln2b(l) + d; }
  int64_t bfc(int l) const { return wfc(l) + 4 * (int64_t)d * d; }
  int64_t wproj(int l) const { return bfc(l) + 4 * (int64_t)d; }
  int64_t bproj(int l) const { return wproj(l) + 4 * (int64_t)d * d; }
};

bool validate(const gpt2_config* c, std::string& why) {
  if (!c) { why = "config is NULL"; return false; }
  if (c->n_layer < 1 || c->d_model < 1 || c->n_head < 1 || c->seq_len < 1 || c->batch < 1) {
    why = "n_layer, d_model, n_head, seq_len and batch must be >= 1"; return false;
  }
  if (c->d_model % c->n_head) { why = "d_model must be divisible by n_head"; return false; }
  if (c->vocab < 1 || c->vocab_padded < c->vocab) { why = "need 1 <= vocab <= vocab_padded"; return false; }
  if (c->vocab_padded > 65536) { why = "vocab_padded must be <= 65536"; return false; }
  if (c->precision != GPT2_FP32 && c->precision != GPT2_BF16) { why = "unknown precision"; return false; }
  if (c->reserved != 0) { why = "reserved must be 0"; return false; }
  if (!(c->init_std >= 0.0f) || !isfinite(c->init_std)) { why = "init_std must be finite and >= 0"; return false; }
  return true;
}

// Valid but outside the kernels' coverage.
bool supported(const gpt2_config* c, std::string& why) {
  const int hd = c->d_model / c->n_head;
  if (hd != 16 && hd != 32 && hd != 64) { why = "head_dim must be 16, 32 or 64"; return false; }
  if (c->d_model % 8) { why = "d_model must be a multiple of 8"; return false; }
  if (c->d_model > 2048) { why = "d_model must be <= 2048"; return false; }
  if (c->vocab_padded % 8) { why = "vocab_padded must be a multiple of 8"; return false; }
  if ((int64_t)c->batch * c->seq_len > MAX_ROWS) { why = "batch * seq_len must be <= 65536"; return false; }
  if (c->precision == GPT2_FP32 && c->vocab_padded > 32768) {
    why = "fp32 precision supports vocab_padded <= 32768"; return false;
  }
  return true;
}

Geo geometry(const gpt2_config* c) {
  Geo g;
  g.L = c->n_layer; g.d = c->d_model; g.H = c->n_head; g.hd = g.d / g.H;
  g.T = c->seq_len; g.B = c->batch; g.M = g.B * g.T; g.V = c->vocab; g.Vp = c->vocab_padded;
  g.bf16 = c->precision == GPT2_BF16;
  const int64_t d = g.d;
  g.P_layer = 12 * d * d + 13 * d;
  g.wte = 0;
  g.wpe = (int64_t)g.Vp * d;
  g.layer0 = g.wpe + (int64_t)g.T * d;
  g.lnfg = g.layer0 + g.L * g.P_layer;
  g.lnfb = g.lnfg + d;
  g.N = g.lnfb + d;
  return g;
}

// Tensors in canonical order: (offset, count, is_matrix, is_ln_gain)
struct Tensor { int64_t off, count; bool matrix, gain; };
std::vector<Tensor> tensors(const Geo& g) {
  std::vector<Tensor> t;
  const int64_t d = g.d;
  t.push_back({g.wte, (int64_t)g.Vp * d, true, false});
  t.push_back({g.wpe, (int64_t)g.T * d, true, false});
  for (int l = 0; l < g.L; ++l) {
    t.push_back({g.ln1g(l), d, false, true});
    t.push_back({g.ln1b(l), d, false, false});
    t.push_back({g.wqkv(l), 3 * d * d, true, false});
    t.push_back({g.bqkv(l), 3 * d, false, false});
    t.push_back({g.wo(l), d * d, true, false});
    t.push_back({g.bo(l), d, false, false});
    t.push_back({g.ln2g(l), d, false, true});
    t.push_back({g.ln2b(l), d, false, false});
    t.push_back({g.wfc(l), 4 * d * d, true, false});
    t.push_back({g.bfc(l), 4 * d, false, false});
    t.push_back({g.wproj(l), 4 * d * d, true, false});
    t.push_back({g.bproj(l), d, false, false});
  }
  t.push_back({g.lnfg, d, false, true});
  t.push_back({g.lnfb, d, false, false});
  return t;
}

std::vector<AdamSeg> decay_segments(const Geo& g) {
  std::vector<AdamSeg> s;
  for (const Tensor& t : tensors(g)) {
    const int dec = t.matrix ? 1 : 0;
    if (s.empty() || s.back().decay != dec) s.push_back({t.off, dec, 0});
  }
  return s;
}

// ------------------------------------------------------------------------------ GEMM plans
// Tile choice measured on the GPT-2 shapes: 256x256 tiles only when they still give at least two
// rounds of blocks over the 256 CUs; otherwise 128x128 tiles (several blocks per CU).
// The GELU-backward product also sums its output columns when it takes the direct-to-LDS bf16
// path (K = d a multiple of 64, leading dimensions well inside 32-bit offsets).
bool fused_colsum(const Geo& g) { return g.bf16 && g.d % 64 == 0 && 4 * g.d < (1 << 22); }

int pick_tile(const Geo& g, int M, int N) {
  if (!g.bf16) return TILE_128;
  return gemm_pick_tile(M, N);
}

// Split of the K = rows reduction of a weight gradient (in x out, K = tokens); the fp32 partials
// are summed by a second kernel in a fixed order. bf16 runs 256x256 tiles at one block per CU and
// the splits aim at about 160 blocks, fewer than the 256 CUs: these products run on the side
// stream, and the CUs they leave free take the main stream's LayerNorm, attention and
// input-gradient kernels, which otherwise wait for whole products to drain (step time measured
// with targets 256, 224, 192, 160, 128, 96 and 64 blocks: 160 best, 1.5% below 256; 96 and
// fewer leave the weight gradients on the critical path). fp32 runs 128x128 tiles and aims at
// about 1024 blocks.
struct Split { int splits, k_split; };
Split pick_split(const Geo& g, int in, int out) {
  const int kt = 64;
  int s;
  if (g.bf16) {
    const int64_t tiles = (int64_t)((in + 255) / 256) * ((out + 255) / 256);
    s = (int)(160 / tiles);
    if (s > 16) s = 16;
  } else {
    const int64_t tiles = (int64_t)((in + 127) / 128) * ((out + 127) / 128);
    s = (int)((1024 + tiles - 1) / tiles);
    if (s > 8) s = 8;
  }
  if (s < 1) s = 1;
  int per = (g.M + s - 1) / s;
  per = (per + kt - 1) / kt * kt;
  if (per < kt) per = kt;
  s = (g.M + per - 1) / per;
  return {s, per};
}

// Splits of the LM head's input gradient dz wte (K = Vp, long): 256 x 256 output tiles, with the
// split count (1..8) whose work items fill whole rounds of the chip's 256 CUs best (fewest rounds
// per unit of work, ties to fewer splits); one split, and the default tiles, on the fp32 path or
// where the vocabulary is not a whole number of 64-wide k-slabs. At GPT-2 124M (192 tiles) four
// splits make three full rounds: 15 % faster than one pass of 128 x 384 tiles, partial sums
// included.
Split lm_dx_split(const Geo& g) {
  if (!g.bf16 || g.Vp % 64) return {1, g.Vp};
  const int64_t tiles = (int64_t)((g.M + 255) / 256) * ((g.d + 255) / 256);
  int best = 1;
  int64_t best_rounds = (tiles + 255) / 256;  // compared as rounds / splits
  for (int s = 2; s <= 8; ++s) {
    const int64_t rounds = (tiles * s + 255) / 256;
    if (rounds * best < best_rounds * s) {
      best = s;
      best_rounds = rounds;
    }
  }
  int per = (g.Vp + best - 1) / best;
  per = (per + 63) / 64 * 64;
  return {(g.Vp + per - 1) / per, per};
}

// Column sums of the backward (bias, LayerNorm gain and shift gradients): every reduction writes
// its partial rows to a slice of its own and all are summed by one batched launch at the end
// of the backward (49 launches of a few microseconds each before). Slices: LayerNorm k = 2l
// (ln1 of layer l), 2l + 1 (ln2), 2L (final); then the QKV bias per layer; then the fc bias.
struct ColLayout {
  size_t ln, qkv, fc, total;  // floats per slice, and in all
  int nparts_ln, nparts_qkv, nparts_fc, ntasks;
};
ColLayout col_layout(const Geo& g) {
  ColLayout cl{};
  const size_t d = g.d;
  cl.nparts_ln = ln_bwd_blocks(g.M, LN_ROWS_PER_BLOCK);
  cl.nparts_qkv = (g.M + COLSUM_ROWS_PER_BLOCK - 1) / COLSUM_ROWS_PER_BLOCK;
  if (fused_colsum(g)) {
    // rows per block of the product that writes the partial rows (128 x 384 tiles fall back to
    // 256 x 256 when column sums are asked for)
    const int bm = pick_tile(g, g.M, 4 * g.d) == TILE_128 ? 128 : 256;
    cl.nparts_fc = 2 * ((g.M + bm - 1) / bm);
  } else {
    cl.nparts_fc = cl.nparts_qkv;
  }
  cl.ln = (size_t)cl.nparts_ln * 3 * d;
  cl.qkv = (size_t)cl.nparts_qkv * 3 * d;
  cl.fc = (size_t)cl.nparts_fc * 4 * d;
  cl.total = (2 * (size_t)g.L + 1) * cl.ln + (size_t)g.L * (cl.qkv + cl.fc);
  cl.ntasks = 4 * g.L + 1;
  return cl;
}

// ------------------------------------------------------------------------------ buffers
struct Bufs {
  float *params = nullptr, *grads = nullptr, *m = nullptr, *v = nullptr;
  void* shadow = nullptr;
  std::vector<float*> resid, resid_mid, ln1_mean, ln1_rstd, ln2_mean, ln2_rstd, lse;
  std::vector<void*> ln1, qkv, att, ln2, fc, act;
  void* lnf = nullptr;
  float *lnf_mean = nullptr, *lnf_rstd = nullptr;
  void* logits = nullptr;
  float *row_loss = nullptr, *loss = nullptr;
  int* err = nullptr;
  float* dres = nullptr;
  // Output gradients that weight-gradient products read on the side stream get a buffer per
  // producer, so the backward on the main stream never overwrites one still being read:
  // dres_t per LayerNorm backward (slot k as for the column sums), dbig and dqkv per layer.
  std::vector<void*> dres_t, dbig, dqkv;
  float* dtmp = nullptr;
  void* datt = nullptr;
  float* dsum = nullptr;
  float* colpart = nullptr;      // column-sum partial rows: one slice per reduction of a backward
  ColTask* coltasks = nullptr;   // the reductions of those slices (device table, built at init)
  int ncoltasks = 0, ncolblocks = 0;
  float* splitk = nullptr;
  float* lmdx_part = nullptr;  // fp32 split partials of the LM head's input gradient
  uint32_t* keys = nullptr;
  float* segpart = nullptr;
  float* clip = nullptr;  // gradient-norm block sums, the norm and the clipping factor
};

struct Carver {
  uintptr_t base;
  size_t off = 0;
  template <typename P>
  P* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    P* p = reinterpret_cast<P*>(base + off);
    off += bytes;
    return p;
  }
};

size_t carve(const Geo& g, uintptr_t base, Bufs& b) {
  Carver c{base};
  const size_t ts = g.bf16 ? 2 : 4;
  const size_t N = (size_t)g.N, M = (size_t)g.M, d = (size_t)g.d;
  b.params = c.take<float>(4 * N);
  b.grads = c.take<float>(4 * N);
  b.m = c.take<float>(4 * N);
  b.v = c.take<float>(4 * N);
  b.shadow = g.bf16 ? c.take<void>(2 * N) : nullptr;
  const size_t bht = (size_t)g.B * g.H * g.T;
  b.resid.resize(g.L + 1);
  b.resid_mid.resize(g.L);
  b.ln1.resize(g.L); b.qkv.resize(g.L); b.att.resize(g.L); b.ln2.resize(g.L);
  b.fc.resize(g.L); b.act.resize(g.L);
  b.ln1_mean.resize(g.L); b.ln1_rstd.resize(g.L); b.ln2_mean.resize(g.L); b.ln2_rstd.resize(g.L);
  b.lse.resize(g.L);
  for (int l = 0; l <= g.L; ++l) b.resid[l] = c.take<float>(4 * M * d);
  for (int l = 0; l < g.L; ++l) {
    b.resid_mid[l] = c.take<float>(4 * M * d);
    b.ln1[l] = c.take<void>(ts * M * d);
    b.ln1_mean[l] = c.take<float>(4 * M);
    b.ln1_rstd[l] = c.take<float>(4 * M);
    b.qkv[l] = c.take<void>(ts * M * 3 * d);
    b.att[l] = c.take<void>(ts * M * d);
    b.lse[l] = c.take<float>(4 * bht);
    b.ln2[l] = c.take<void>(ts * M * d);
    b.ln2_mean[l] = c.take<float>(4 * M);
    b.ln2_rstd[l] = c.take<float>(4 * M);
    b.fc[l] = c.take<void>(ts * M * 4 * d);
    b.act[l] = c.take<void>(ts * M * 4 * d);
  }
  b.lnf = c.take<void>(ts * M * d);
  b.lnf_mean = c.take<float>(4 * M);
  b.lnf_rstd = c.take<float>(4 * M);
  b.logits = c.take<void>(ts * M * (size_t)g.Vp);
  b.row_loss = c.take<float>(4 * M);
  b.loss = c.take<float>(8);  // mean loss, 1 / (number of trained positions)
  b.err = c.take<int>(4);
  b.dres = c.take<float>(4 * M * d);
  b.dres_t.resize(2 * g.L + 1);
  for (auto& p : b.dres_t) p = c.take<void>(ts * M * d);
  b.dtmp = c.take<float>(4 * M * d);
  b.dbig.resize(g.L);
  for (auto& p : b.dbig) p = c.take<void>(ts * M * 4 * d);
  b.dqkv.resize(g.L);
  for (auto& p : b.dqkv) p = c.take<void>(ts * M * 3 * d);
  b.datt = c.take<void>(ts * M * d);
  b.dsum = c.take<float>(8 * bht);  // attention backward scratch: 2 floats per (b, h, t)
  const size_t nblk = (size_t)ln_bwd_blocks(g.M, LN_ROWS_PER_BLOCK);
  const size_t ncs = (M + COLSUM_ROWS_PER_BLOCK - 1) / COLSUM_ROWS_PER_BLOCK;
  (void)nblk;
  (void)ncs;
  const ColLayout cl = col_layout(g);
  b.colpart = c.take<float>(4 * cl.total);
  b.coltasks = c.take<ColTask>(sizeof(ColTask) * cl.ntasks);
  size_t sk = 0;
  const int shapes[4][2] = {{g.d, 3 * g.d}, {g.d, g.d}, {g.d, 4 * g.d}, {4 * g.d, g.d}};
  for (auto& s : shapes) {
    const Split sp = pick_split(g, s[0], s[1]);
    if (sp.splits > 1) sk = std::max(sk, (size_t)sp.splits * s[0] * s[1]);
  }
  b.splitk = c.take<float>(4 * std::max<size_t>(sk, 1));
  const Split lsp = lm_dx_split(g);
  if (lsp.splits > 1) b.lmdx_part = c.take<float>(4 * (size_t)lsp.splits * M * d);
  b.keys = c.take<uint32_t>(4 * M);
  b.segpart = c.take<float>(4 * (size_t)embed_bwd_chunks(g.M) * 2 * d);
  b.clip = c.take<float>(4 * (size_t)(CLIP_PARTS + 4));
  return (c.off + 255) & ~(size_t)255;
}

}  // namespace

// ------------------------------------------------------------------------------ context
namespace {
float* ln_part(const Geo& g, const Bufs& b, int k) { return b.colpart + (size_t)k * col_layout(g).ln; }
float* qkv_part(const Geo& g, const Bufs& b, int l) {
  const ColLayout cl = col_layout(g);
  return b.colpart + (2 * (size_t)g.L + 1) * cl.ln + (size_t)l * cl.qkv;
}
float* fc_part(const Geo& g, const Bufs& b, int l) {
  const ColLayout cl = col_layout(g);
  return b.colpart + (2 * (size_t)g.L + 1) * cl.ln + (size_t)g.L * cl.qkv + (size_t)l * cl.fc;
}

// The backward's column reductions over those slices (in any order: their outputs are disjoint)
std::vector<ColTask> col_tasks(const Geo& g, const Bufs& b) {
  const ColLayout cl = col_layout(g);
  float* G = b.grads;
  const int d = g.d;
  std::vector<ColTask> t;
  auto add = [&](const float* part, int nparts, int64_t stride, int seg, float* o0, float* o1,
                 float* o2) {
    const int nseg = o2 ? 3 : (o1 ? 2 : 1);
    t.push_back(ColTask{part, stride, nparts, nseg * seg, seg, 0, {o0, o1, o2}});
  };
  add(ln_part(g, b, 2 * g.L), cl.nparts_ln, 3 * d, d, G + g.lnfg, G + g.lnfb, G + g.bproj(g.L - 1));
  for (int l = g.L - 1; l >= 0; --l) {
    add(fc_part(g, b, l), cl.nparts_fc, 4 * d, 4 * d, G + g.bfc(l), nullptr, nullptr);
    add(ln_part(g, b, 2 * l + 1), cl.nparts_ln, 3 * d, d, G + g.ln2g(l), G + g.ln2b(l), G + g.bo(l));
    add(qkv_part(g, b, l), cl.nparts_qkv, 3 * d, 3 * d, G + g.bqkv(l), nullptr, nullptr);
    add(ln_part(g, b, 2 * l), cl.nparts_ln, 3 * d, d, G + g.ln1g(l), G + g.ln1b(l),
        l > 0 ? G + g.bproj(l - 1) : nullptr);
  }
  int blk = 0;
  for (ColTask& k : t) {
    k.block0 = blk;
    blk += (k.n + 63) / 64;
  }
  return t;
}
}  // namespace

struct gpt2_ctx {
  gpt2_config cfg;
  Geo g;
  Bufs b;
  hipStream_t stream;
  // side stream for work off the forward's critical path (the token sort), joined by events
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr, tail = nullptr;
  hipEvent_t wte_dw = nullptr;  // the LM head's (tied) weight gradient is written
  // backward: LayerNorm slot k done (2L + 1), dbig and dqkv of layer l written (L each)
  std::vector<hipEvent_t> ev_ln, ev_dbig, ev_dqkv;
  // AdamW: parameter range r updated (embeddings, layers 0 .. L-1, final LayerNorm: L + 2)
  std::vector<hipEvent_t> ev_adam;
  int64_t t = 0;
  bool have_forward = false;
  bool in_backward = false;  // which phase a matrix product belongs to (timing families)
  std::vector<AdamSeg> segs;
  // timing
  int timing_family = -1;
  std::vector<hipEvent_t> ev;
  int timed = 0;
  double timed_work = 0.0;
};

namespace {

// Records an event pair around one launch when its family is being timed.
struct Timed {
  gpt2_ctx* c;
  hipStream_t s;
  bool on;
  Timed(gpt2_ctx* c_, int family, double work, hipStream_t s_ = nullptr)
      : c(c_), s(s_ ? s_ : c_->stream), on(false) {
    if (c->timing_family == family && c->timed < TIMING_CAP) {
      on = true;
      hipEventRecord(c->ev[2 * c->timed], s);
      c->timed_work += work;
    }
  }
  void stop() {
    if (on) {
      hipEventRecord(c->ev[2 * c->timed + 1], s);
      ++c->timed;
      on = false;
    }
  }
  ~Timed() { stop(); }
};

// Kernel families that gpt2_timing_begin can time (the numbering is the ABI's).
enum {
  FAM_LMHEAD = 0,     // LM-head forward product
  FAM_GEMM = 1,       // every matrix product
  FAM_ATTN = 2,       // attention forward
  FAM_XENT = 3,       // fused cross-entropy
  FAM_ADAMW = 4,      // AdamW
  FAM_DW = 5,         // weight-gradient products (incl. the tied LM head's)
  FAM_ATTN_BWD = 6,   // attention backward (dK/dV and dQ kernels)
  FAM_LN_FWD = 7,     // LayerNorm forward
  FAM_LN_BWD = 8,     // LayerNorm backward
  FAM_SPLITK = 9,     // split-K partial sums of the weight gradients
  FAM_COLSUM = 10,    // bias / LayerNorm parameter column sums (partials and the batched sum)
  FAM_EMBED = 11,     // embedding gather, token sort and embedding backward
  FAM_GEMM_FWD = 12,  // forward products (incl. the LM head)
  FAM_GEMM_DX = 13,   // input-gradient products
  FAM_COUNT = 14
};

const void* W(gpt2_ctx* c, int64_t off) {
  return c->g.bf16 ? (const void*)(static_cast<const char*>(c->b.shadow) + 2 * off)
                   : (const void*)(c->b.params + off);
}

gpt2_status gemm(gpt2_ctx* c, int a_kmajor, int b_kmajor, int M, int N, int K, const void* A,
                 int64_t lda, const void* B, int64_t ldb, int epi, void* C, int64_t ldc,
                 const float* bias = nullptr, const float* resid = nullptr, void* C2 = nullptr,
                 const void* aux = nullptr, float alpha = 1.0f, float beta = 0.0f, int tag = 0,
                 float* colsum = nullptr, const float* alpha_scale = nullptr) {
  GemmParams p{};
  p.A = A; p.lda = lda; p.B = B; p.ldb = ldb;
  p.M = M; p.N = N; p.K = K; p.k_split = K;
  p.epi = epi; p.C = C; p.ldc = ldc; p.c_split_stride = 0;
  p.C2 = C2; p.bias = bias; p.resid = resid; p.aux = aux; p.alpha = alpha; p.beta = beta;
  p.colsum = colsum;
  p.alpha_scale = alpha_scale;
  const double fl = 2.0 * M * N * K;
  Timed t1(c, FAM_GEMM, fl);
  Timed t0(c, tag == 1 ? FAM_LMHEAD : -2, fl);
  Timed t2(c, c->in_backward ? FAM_GEMM_DX : FAM_GEMM_FWD, fl);
  const int tile = c->g.bf16
                       ? gemm_pick_tile_epi(M, N, a_kmajor, b_kmajor, epi, colsum != nullptr)
                       : TILE_128;
  HIPCHK(launch_gemm(c->g.bf16, a_kmajor, b_kmajor, tile, 1, tag, p, c->stream));
  return GPT2_OK;
}

// Weight gradient dW (in x out) = X^T dY over the M rows, X (M x in) and dY (M x out) row-major,
// written (accumulate = 0) or added (1) into the fp32 gradient at gw.
gpt2_status gemm_dw(gpt2_ctx* c, int in, int out, const void* X, const void* dY, float* gw,
                    int accumulate, hipStream_t st) {
  const Geo& g = c->g;
  const Split sp = pick_split(g, in, out);
  GemmParams p{};
  p.A = X; p.lda = in; p.B = dY; p.ldb = out;
  p.M = in; p.N = out; p.K = g.M; p.k_split = sp.k_split;
  p.epi = EPI_F32; p.alpha = 1.0f;
  Timed t1(c, FAM_GEMM, 2.0 * in * out * g.M, st);
  Timed t2(c, FAM_DW, 2.0 * in * out * g.M, st);
  const int tile = g.bf16 ? TILE_256 : TILE_128;
  if (sp.splits == 1) {
    p.C = gw; p.ldc = out; p.beta = accumulate ? 1.0f : 0.0f;
    HIPCHK(launch_gemm(g.bf16, 0, 0, tile, 1, 0, p, st));
  } else {
    p.C = c->b.splitk; p.ldc = out; p.c_split_stride = (int64_t)in * out; p.beta = 0.0f;
    HIPCHK(launch_gemm(g.bf16, 0, 0, tile, sp.splits, 0, p, st));
    t2.stop();
    t1.stop();
    // reads the splits' fp32 partials, writes (and when accumulating reads) the gradient
    Timed t3(c, FAM_SPLITK, 4.0 * in * out * (sp.splits + 1 + (accumulate ? 1 : 0)), st);
    HIPCHK(launch_splitk_reduce(c->b.splitk, sp.splits, (int64_t)in * out, in, out, gw, out, 1.0f,
                                accumulate ? 1.0f : 0.0f, st));
  }
  return GPT2_OK;
}

// Column partial sums of an (M, N) matrix into `part` (reduced with the others at the end)
gpt2_status colsum(gpt2_ctx* c, const void* src, int N, float* part, hipStream_t st) {
  const Geo& g = c->g;
  Timed t(c, FAM_COLSUM, (double)(g.bf16 ? 2 : 4) * g.M * N, st);
  HIPCHK(launch_colsum_partial(g.bf16, g.M, N, src, N, part, COLSUM_ROWS_PER_BLOCK, st));
  return GPT2_OK;
}

// LayerNorm backward into the residual gradient; its three column partial sums (gain and shift
// gradients, and the bias gradient of the projection that produced this residual stream) go to
// LayerNorm slice k and are reduced with the others at the end of the backward.
// LayerNorm backward of slot k; its launch records ev_ln[k] for the side stream.
gpt2_status ln_backward(gpt2_ctx* c, const float* x, const float* mean, const float* rstd,
                        int64_t g_off, int has_dres, int k) {
  const Geo& g = c->g;
  // reads dy (bf16 or fp32), x and the incoming residual gradient (fp32); writes the residual
  // gradient (fp32) and its copy in the product's element type
  const double es = g.bf16 ? 2.0 : 4.0;
  Timed t(c, FAM_LN_BWD, ((double)g.M * g.d) * (es + 4.0 + (has_dres ? 4.0 : 0.0) + 4.0 + es));
  HIPCHK(launch_ln_bwd(g.bf16, g.M, g.d, c->b.dtmp, x, mean, rstd, c->b.params + g_off, c->b.dres,
                       has_dres, c->b.dres_t[k], ln_part(g, c->b, k), LN_ROWS_PER_BLOCK,
                       c->stream, c->ev_ln[k]));
  return GPT2_OK;
}

// LayerNorm forward of the residual stream x into y (bf16 or fp32) and its row statistics
gpt2_status ln_forward(gpt2_ctx* c, const float* x, int64_t g_off, int64_t b_off, void* y,
                       float* mean, float* rstd) {
  const Geo& g = c->g;
  // reads x (fp32), writes y
  Timed t(c, FAM_LN_FWD, (double)g.M * g.d * (4.0 + (g.bf16 ? 2.0 : 4.0)));
  HIPCHK(launch_ln_fwd(g.bf16, g.M, g.d, x, c->b.params + g_off, c->b.params + b_off, y, mean,
                       rstd, c->stream));
  return GPT2_OK;
}

#define STEP(x)                          \
  do {                                   \
    gpt2_status s_ = (x);                \
    if (s_ != GPT2_OK) return s_;        \
  } while (0)

gpt2_status forward(gpt2_ctx* c, const int32_t* tokens, const int32_t* targets, float* loss_user) {
  const Geo& g = c->g;
  Bufs& b = c->b;
  float* P = b.params;
  const int M = g.M, d = g.d;
  // each parameter range is used once the last AdamW step has updated it (events of the side
  // stream; recorded already when no update is pending)
  HIPCHK(hipStreamWaitEvent(c->stream, c->ev_adam[0], 0));
  {
    Timed t(c, FAM_EMBED, 0.0);
    HIPCHK(launch_embed_fwd(g.B, g.T, d, g.V, tokens, P + g.wte, P + g.wpe, b.resid[0], b.err,
                            c->stream));
  }
  // The token sort (one workgroup, ~150 us) feeds only the embedding backward: it runs on the side
  // stream beside the forward's kernels, and the end of the forward waits for it.
  HIPCHK(hipEventRecord(c->fork, c->stream));
  HIPCHK(hipStreamWaitEvent(c->side, c->fork, 0));
  {
    Timed t(c, FAM_EMBED, 0.0, c->side);
    HIPCHK(launch_token_sort(M, g.V, tokens, b.keys, c->side));
  }
  HIPCHK(hipEventRecord(c->join, c->side));
  for (int l = 0; l < g.L; ++l) {
    HIPCHK(hipStreamWaitEvent(c->stream, c->ev_adam[1 + l], 0));
    STEP(ln_forward(c, b.resid[l], g.ln1g(l), g.ln1b(l), b.ln1[l], b.ln1_mean[l],
                    b.ln1_rstd[l]));
    STEP(gemm(c, 1, 0, M, 3 * d, d, b.ln1[l], d, W(c, g.wqkv(l)), 3 * d, EPI_STORE, b.qkv[l],
              3 * d, P + g.bqkv(l)));
    {
      Timed t(c, FAM_ATTN, 4.0 * g.B * g.H * g.hd * ((double)g.T * (g.T + 1) / 2));
      HIPCHK(launch_attn_fwd(g.bf16, g.B, g.T, g.H, g.hd, b.qkv[l], b.att[l], b.lse[l],
                             c->stream));
    }
    STEP(gemm(c, 1, 0, M, d, d, b.att[l], d, W(c, g.wo(l)), d, EPI_BIAS_RESID, b.resid_mid[l], d,
              P + g.bo(l), b.resid[l]));
    STEP(ln_forward(c, b.resid_mid[l], g.ln2g(l), g.ln2b(l), b.ln2[l], b.ln2_mean[l],
                    b.ln2_rstd[l]));
    STEP(gemm(c, 1, 0, M, 4 * d, d, b.ln2[l], d, W(c, g.wfc(l)), 4 * d, EPI_BIAS_GELU, b.fc[l],
              4 * d, P + g.bfc(l), nullptr, b.act[l]));
    STEP(gemm(c, 1, 0, M, d, 4 * d, b.act[l], 4 * d, W(c, g.wproj(l)), d, EPI_BIAS_RESID,
              b.resid[l + 1], d, P + g.bproj(l), b.resid_mid[l]));
  }
  HIPCHK(hipStreamWaitEvent(c->stream, c->ev_adam[g.L + 1], 0));
  STEP(ln_forward(c, b.resid[g.L], g.lnfg, g.lnfb, b.lnf, b.lnf_mean, b.lnf_rstd));
  STEP(gemm(c, 1, 1, M, g.Vp, d, b.lnf, d, W(c, g.wte), d, EPI_STORE, b.logits, g.Vp, nullptr,
            nullptr, nullptr, nullptr, 1.0f, 0.0f, 1));
  {
    const double bytes = 2.0 * (g.bf16 ? 2 : 4) * (double)M * g.Vp;
    Timed t(c, FAM_XENT, bytes);
    HIPCHK(launch_xent(g.bf16, M, g.V, g.Vp, b.logits, targets, b.row_loss, b.err, c->stream));
  }
  HIPCHK(launch_loss_mean(M, b.row_loss, targets, b.loss, loss_user, c->stream));
  HIPCHK(hipStreamWaitEvent(c->stream, c->join, 0));  // the sort has read the tokens
  return GPT2_OK;
}

// The backward runs the chain of input gradients (the critical path) on the main stream and
// every weight-gradient product (with its split-K sum) and the QKV bias partial sums on the side
// stream, each waiting for the event of the output gradient it reads. The two streams fill each
// other's idle CUs (a product's partly filled last round of tiles, the latency-bound attention
// backward). The embedding backward, which adds to the LM head's weight gradient, waits for that
// product only; the main stream joins the whole side stream before the backward returns.
gpt2_status backward(gpt2_ctx* c, float grad_scale, int acc) {
  const Geo& g = c->g;
  Bufs& b = c->b;
  float* G = b.grads;
  const int M = g.M, d = g.d;
  // the LM-head gradient products scale by grad_scale / n, n = the number of trained positions
  // (all M unless targets are -1), which the loss-mean kernel left on the device
  const float* inv_n = b.loss + 1;
  hipStream_t side = c->side;
  // every AdamW range has landed (a forward normally waited for them already)
  HIPCHK(hipStreamWaitEvent(c->stream, c->ev_adam[g.L + 1], 0));
  HIPCHK(hipEventRecord(c->fork, c->stream));  // the logits' gradients (cross-entropy) are done
  HIPCHK(hipStreamWaitEvent(side, c->fork, 0));
  // LM head (tied), s = grad_scale / n: dwte = s * dz^T lnf (+ existing when accumulating), on
  // the side stream; df = s * dz wte. The input gradients that feed a LayerNorm backward (dtmp) are bf16 on the
  // bf16 path, as a bf16 product's output gradient is in mixed-precision training; fp32 otherwise.
  {
    GemmParams p{};
    p.A = b.logits; p.lda = g.Vp; p.B = b.lnf; p.ldb = d;
    p.M = g.Vp; p.N = d; p.K = M; p.k_split = M;
    p.epi = EPI_F32; p.C = G + g.wte; p.ldc = d; p.alpha = grad_scale; p.beta = acc ? 1.0f : 0.0f;
    p.alpha_scale = inv_n;
    Timed t(c, FAM_GEMM, 2.0 * g.Vp * d * M, side);
    Timed t2(c, FAM_DW, 2.0 * g.Vp * d * M, side);
    HIPCHK(launch_gemm(g.bf16, 0, 0, pick_tile(g, g.Vp, d), 1, 0, p, side));
    t2.stop();
    t.stop();
    HIPCHK(hipEventRecord(c->wte_dw, side));
  }
  const int epi_dy = g.bf16 ? EPI_STORE : EPI_F32;
  const Split lsp = lm_dx_split(g);
  if (lsp.splits > 1) {
    // fp32 partials of K-splits, then their sum in split order, scaled by s, rounded to bf16
    GemmParams p{};
    p.A = b.logits; p.lda = g.Vp; p.B = W(c, g.wte); p.ldb = d;
    p.M = M; p.N = d; p.K = g.Vp; p.k_split = lsp.k_split;
    p.epi = EPI_F32; p.C = b.lmdx_part; p.ldc = d; p.c_split_stride = (int64_t)M * d;
    p.alpha = 1.0f; p.beta = 0.0f;
    const double fl = 2.0 * M * d * g.Vp;
    {
      Timed t1(c, FAM_GEMM, fl);
      Timed t2(c, FAM_GEMM_DX, fl);
      HIPCHK(launch_gemm(true, 1, 0, TILE_256, lsp.splits, 0, p, c->stream));
    }
    // reads the splits' fp32 partials, writes the bf16 input gradient
    Timed t3(c, FAM_SPLITK, (4.0 * lsp.splits + 2.0) * M * d);
    HIPCHK(launch_splitk_reduce_bf16(b.lmdx_part, lsp.splits, (int64_t)M * d, M, d, b.dtmp, d,
                                     grad_scale, inv_n, c->stream));
  } else {
    STEP(gemm(c, 1, 0, M, d, g.Vp, b.logits, g.Vp, W(c, g.wte), d, epi_dy, b.dtmp, d, nullptr,
              nullptr, nullptr, nullptr, grad_scale, 0.0f, 0, nullptr, inv_n));
  }
  STEP(ln_backward(c, b.resid[g.L], b.lnf_mean, b.lnf_rstd, g.lnfg, 0, 2 * g.L));
  for (int l = g.L - 1; l >= 0; --l) {
    // h_{l+1} = h_mid + act W_proj + b_proj: its gradient came from LayerNorm slot kp
    const int kp = l == g.L - 1 ? 2 * g.L : 2 * (l + 1);
    void* dh = b.dres_t[kp];
    HIPCHK(hipStreamWaitEvent(side, c->ev_ln[kp], 0));
    STEP(gemm_dw(c, 4 * d, d, b.act[l], dh, G + g.wproj(l), acc, side));
    // du = (dh W_proj^T) o GELU'(u); its column sums (the fc bias gradient) come out of the same
    // product's epilogue as one partial row per 128 (or 64) rows when it runs the direct-to-LDS
    // bf16 path, else from a separate pass
    if (fused_colsum(g)) {
      STEP(gemm(c, 1, 1, M, 4 * d, d, dh, d, W(c, g.wproj(l)), d, EPI_GELU_BWD, b.dbig[l],
                4 * d, nullptr, nullptr, nullptr, b.fc[l], 1.0f, 0.0f, 0, fc_part(g, b, l)));
    } else {
      STEP(gemm(c, 1, 1, M, 4 * d, d, dh, d, W(c, g.wproj(l)), d, EPI_GELU_BWD, b.dbig[l],
                4 * d, nullptr, nullptr, nullptr, b.fc[l]));
      STEP(colsum(c, b.dbig[l], 4 * d, fc_part(g, b, l), c->stream));
    }
    HIPCHK(hipEventRecord(c->ev_dbig[l], c->stream));
    HIPCHK(hipStreamWaitEvent(side, c->ev_dbig[l], 0));
    STEP(gemm_dw(c, d, 4 * d, b.ln2[l], b.dbig[l], G + g.wfc(l), acc, side));
    STEP(gemm(c, 1, 1, M, d, 4 * d, b.dbig[l], 4 * d, W(c, g.wfc(l)), 4 * d, epi_dy, b.dtmp, d));
    STEP(ln_backward(c, b.resid_mid[l], b.ln2_mean[l], b.ln2_rstd[l], g.ln2g(l), 1, 2 * l + 1));
    // h_mid = h_l + att W_o + b_o
    void* dm = b.dres_t[2 * l + 1];
    HIPCHK(hipStreamWaitEvent(side, c->ev_ln[2 * l + 1], 0));
    STEP(gemm_dw(c, d, d, b.att[l], dm, G + g.wo(l), acc, side));
    STEP(gemm(c, 1, 1, M, d, d, dm, d, W(c, g.wo(l)), d, EPI_STORE, b.datt, d));
    {
      // counted work: dV, dP, dQ and dK, each 2 hd FLOPs per causal (query, key) pair
      Timed t(c, FAM_ATTN_BWD, 8.0 * g.B * g.H * g.hd * ((double)g.T * (g.T + 1) / 2));
      HIPCHK(launch_attn_bwd(g.bf16, g.B, g.T, g.H, g.hd, b.qkv[l], b.att[l], b.lse[l], b.datt,
                             b.dqkv[l], b.dsum, c->stream));
    }
    HIPCHK(hipEventRecord(c->ev_dqkv[l], c->stream));
    HIPCHK(hipStreamWaitEvent(side, c->ev_dqkv[l], 0));
    STEP(colsum(c, b.dqkv[l], 3 * d, qkv_part(g, b, l), side));
    STEP(gemm_dw(c, d, 3 * d, b.ln1[l], b.dqkv[l], G + g.wqkv(l), acc, side));
    STEP(gemm(c, 1, 1, M, d, 3 * d, b.dqkv[l], 3 * d, W(c, g.wqkv(l)), 3 * d, epi_dy, b.dtmp, d));
    STEP(ln_backward(c, b.resid[l], b.ln1_mean[l], b.ln1_rstd[l], g.ln1g(l), 1, 2 * l));
  }
  // Every bias and LayerNorm gain/shift gradient from its partial rows, in one launch on the side
  // stream once the last LayerNorm backward has written its rows, beside the embedding backward;
  // the main stream waits for it, and so for all the side stream's work, before the backward
  // ends. The embedding backward adds into the tied wte gradient, so it waits only for the LM
  // head's weight gradient, not for the side stream's last weight gradients.
  HIPCHK(hipStreamWaitEvent(side, c->ev_ln[0], 0));
  {
    Timed t(c, FAM_COLSUM, 4.0 * (double)col_layout(g).total, side);
    HIPCHK(launch_colsum_reduce_batch(b.coltasks, b.ncoltasks, b.ncolblocks, acc, side));
  }
  HIPCHK(hipEventRecord(c->tail, side));
  HIPCHK(hipStreamWaitEvent(c->stream, c->wte_dw, 0));
  Timed te(c, FAM_EMBED, 0.0);
  HIPCHK(launch_embed_bwd(g.B, g.T, d, b.keys, b.dres, G + g.wte, G + g.wpe, acc, b.segpart,
                          c->stream));
  HIPCHK(hipStreamWaitEvent(c->stream, c->tail, 0));
  return GPT2_OK;
}

gpt2_status check_ctx(gpt2_ctx* c) {
  if (!c) return fail(GPT2_E_INVALID, "context is NULL");
  return GPT2_OK;
}

}  // namespace

// ================================================================================== C ABI
extern "C" {

const char* gpt2_last_error(void) { return g_err.c_str(); }

size_t gpt2_workspace_bytes(const gpt2_config* cfg) {
  std::string why;
  if (!validate(cfg, why) || !supported(cfg, why)) return 0;
  Geo g = geometry(cfg);
  Bufs b;
  return carve(g, 0, b);
}

gpt2_status gpt2_param_count(const gpt2_config* cfg, size_t* n) {
  std::string why;
  if (!n) return fail(GPT2_E_INVALID, "n is NULL");
  if (!validate(cfg, why)) return fail(GPT2_E_INVALID, why);
  *n = (size_t)geometry(cfg).N;
  return GPT2_OK;
}

gpt2_status gpt2_init(const gpt2_config* cfg, void* d_arena, size_t arena_bytes, void* hip_stream,
                      gpt2_ctx** out) {
  std::string why;
  if (!out) return fail(GPT2_E_INVALID, "out is NULL");
  *out = nullptr;
  if (!validate(cfg, why)) return fail(GPT2_E_INVALID, why);
  if (!supported(cfg, why)) return fail(GPT2_E_UNSUPPORTED, why);
  if (!d_arena) return fail(GPT2_E_INVALID, "arena is NULL");
  if (reinterpret_cast<uintptr_t>(d_arena) & 255)
    return fail(GPT2_E_INVALID, "arena must be 256-byte aligned");
  const size_t need = gpt2_workspace_bytes(cfg);
  if (arena_bytes < need)
    return fail(GPT2_E_NOMEM, "arena has " + std::to_string(arena_bytes) + " bytes, need " +
                                  std::to_string(need));
  gpt2_ctx* c = new gpt2_ctx();
  c->cfg = *cfg;
  c->g = geometry(cfg);
  c->stream = static_cast<hipStream_t>(hip_stream);
  carve(c->g, reinterpret_cast<uintptr_t>(d_arena), c->b);
  c->segs = decay_segments(c->g);
  const Geo& g = c->g;
  Bufs& b = c->b;
  auto bail = [&](gpt2_status s) {
    if (c->fork) hipEventDestroy(c->fork);
    if (c->join) hipEventDestroy(c->join);
    if (c->tail) hipEventDestroy(c->tail);
    if (c->wte_dw) hipEventDestroy(c->wte_dw);
    for (auto* v : {&c->ev_ln, &c->ev_dbig, &c->ev_dqkv, &c->ev_adam})
      for (hipEvent_t e : *v)
        if (e) hipEventDestroy(e);
    if (c->side) hipStreamDestroy(c->side);
    delete c;
    return s;
  };
#define INITCHK(x)                                                                       \
  do {                                                                                   \
    hipError_t e_ = (x);                                                                 \
    if (e_ != hipSuccess)                                                                \
      return bail(fail(GPT2_E_HIP, std::string(#x) + " failed: " + hipGetErrorString(e_))); \
  } while (0)
  for (const Tensor& t : tensors(g)) {
    if (t.matrix)
      INITCHK(launch_init_normal(t.off, t.count, b.params + t.off, cfg->seed, cfg->init_std,
                                 c->stream));
    else
      INITCHK(launch_fill(t.count, b.params + t.off, t.gain ? 1.0f : 0.0f, c->stream));
  }
  INITCHK(launch_fill(g.N, b.grads, 0.0f, c->stream));
  INITCHK(launch_fill(g.N, b.m, 0.0f, c->stream));
  INITCHK(launch_fill(g.N, b.v, 0.0f, c->stream));
  if (g.bf16) INITCHK(launch_cast_bf16(g.N, b.params, b.shadow, c->stream));
  INITCHK(hipMemsetAsync(b.err, 0, sizeof(int), c->stream));
  INITCHK(hipMemsetAsync(b.loss, 0, 2 * sizeof(float), c->stream));
  const std::vector<ColTask> coltasks = col_tasks(g, b);
  b.ncoltasks = (int)coltasks.size();
  b.ncolblocks = coltasks.empty() ? 0 : coltasks.back().block0 + (coltasks.back().n + 63) / 64;
  INITCHK(hipMemcpyAsync(b.coltasks, coltasks.data(), sizeof(ColTask) * coltasks.size(),
                         hipMemcpyHostToDevice, c->stream));
  INITCHK(hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking));
  INITCHK(hipEventCreateWithFlags(&c->fork, hipEventDisableTiming));
  INITCHK(hipEventCreateWithFlags(&c->join, hipEventDisableTiming));
  INITCHK(hipEventCreateWithFlags(&c->tail, hipEventDisableTiming));
  INITCHK(hipEventCreateWithFlags(&c->wte_dw, hipEventDisableTiming));
  c->ev_ln.assign(2 * g.L + 1, nullptr);
  c->ev_dbig.assign(g.L, nullptr);
  c->ev_dqkv.assign(g.L, nullptr);
  c->ev_adam.assign(g.L + 2, nullptr);
  for (auto* v : {&c->ev_ln, &c->ev_dbig, &c->ev_dqkv, &c->ev_adam})
    for (hipEvent_t& e : *v) INITCHK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  for (hipEvent_t e : c->ev_adam) INITCHK(hipEventRecord(e, c->stream));  // nothing pending
  INITCHK(hipStreamSynchronize(c->stream));
#undef INITCHK
  *out = c;
  return GPT2_OK;
}

gpt2_status gpt2_forward_loss(gpt2_ctx* c, const int32_t* d_tokens, const int32_t* d_targets,
                              float* d_loss) {
  STEP(check_ctx(c));
  if (!d_tokens || !d_targets) return fail(GPT2_E_INVALID, "tokens and targets must not be NULL");
  STEP(forward(c, d_tokens, d_targets, d_loss));
  c->have_forward = true;
  return GPT2_OK;
}

gpt2_status gpt2_backward(gpt2_ctx* c, float grad_scale, int32_t accumulate) {
  STEP(check_ctx(c));
  if (!c->have_forward) return fail(GPT2_E_STATE, "backward needs a forward first");
  if (accumulate != 0 && accumulate != 1) return fail(GPT2_E_INVALID, "accumulate must be 0 or 1");
  if (!isfinite(grad_scale)) return fail(GPT2_E_INVALID, "grad_scale must be finite");
  c->in_backward = true;
  const gpt2_status s = backward(c, grad_scale, accumulate);
  c->in_backward = false;
  return s;
}

gpt2_status gpt2_adamw_step(gpt2_ctx* c, float lr, float beta1, float beta2, float eps,
                            float weight_decay) {
  STEP(check_ctx(c));
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f) || !(eps > 0.0f) ||
      !isfinite(lr) || !isfinite(weight_decay))
    return fail(GPT2_E_INVALID, "need 0 <= beta < 1, eps > 0, finite lr and weight_decay");
  c->t += 1;
  const double bc1 = 1.0 / (1.0 - pow((double)beta1, (double)c->t));
  const double bc2 = 1.0 / (1.0 - pow((double)beta2, (double)c->t));
  // Parameter ranges in the order the forward first uses them: the embeddings, layer 0 .. L-1,
  // the final LayerNorm. Each is updated on the side stream and its event tells the next forward
  // when that range's weights (and their bf16 copy) are ready, so the updates of later layers
  // run beside the forward's first layers.
  const Geo& g = c->g;
  std::vector<int64_t> cut{0, g.layer0};
  for (int l = 1; l <= g.L; ++l) cut.push_back(g.lay(l));
  cut.push_back(g.N);
  bool aligned = true;
  for (int64_t x : cut) aligned = aligned && x % 4 == 0;
  if (!aligned) {
    Timed t(c, FAM_ADAMW, 30.0 * g.N);
    HIPCHK(launch_adamw(0, g.N, c->b.params, c->b.grads, c->b.m, c->b.v, c->b.shadow,
                        c->segs.data(), (int)c->segs.size(), lr, beta1, beta2, eps, weight_decay,
                        (float)bc1, (float)bc2, c->stream));
    for (hipEvent_t e : c->ev_adam) HIPCHK(hipEventRecord(e, c->stream));
    return GPT2_OK;
  }
  HIPCHK(hipEventRecord(c->fork, c->stream));  // the gradients are final
  HIPCHK(hipStreamWaitEvent(c->side, c->fork, 0));
  for (int r = 0; r + 1 < (int)cut.size(); ++r) {
    const int64_t n = cut[r + 1] - cut[r];
    {
      Timed t(c, FAM_ADAMW, 30.0 * n, c->side);
      HIPCHK(launch_adamw(cut[r], n, c->b.params, c->b.grads, c->b.m, c->b.v, c->b.shadow,
                          c->segs.data(), (int)c->segs.size(), lr, beta1, beta2, eps, weight_decay,
                          (float)bc1, (float)bc2, c->side));
    }
    HIPCHK(hipEventRecord(c->ev_adam[r], c->side));
  }
  return GPT2_OK;
}

gpt2_status gpt2_clip_grad_norm(gpt2_ctx* c, float max_norm, float* d_norm) {
  STEP(check_ctx(c));
  if (!(max_norm > 0.0f) || !isfinite(max_norm))
    return fail(GPT2_E_INVALID, "max_norm must be positive and finite");
  // the gradients are final on the main stream (the backward joined its side stream)
  HIPCHK(launch_clip_grad_norm(c->g.N, c->b.grads, max_norm, c->b.clip, d_norm, c->stream));
  return GPT2_OK;
}

gpt2_status gpt2_check(gpt2_ctx* c) {
  STEP(check_ctx(c));
  // the side stream carries AdamW and the weight-gradient products: wait for both streams
  HIPCHK(hipStreamSynchronize(c->stream));
  HIPCHK(hipStreamSynchronize(c->side));
  int err = 0;
  HIPCHK(hipMemcpy(&err, c->b.err, sizeof(int), hipMemcpyDeviceToHost));
  if (err) {
    const int zero = 0;
    HIPCHK(hipMemcpy(c->b.err, &zero, sizeof(int), hipMemcpyHostToDevice));
    std::string what;
    if (err & ERR_TOKEN_RANGE) what += "token id outside [0, vocab); ";
    if (err & ERR_TARGET_RANGE) what += "target id outside [0, vocab) and not -1; ";
    return fail(GPT2_E_DEVICE, what);
  }
  return GPT2_OK;
}

gpt2_status gpt2_destroy(gpt2_ctx* c) {
  if (!c) return fail(GPT2_E_INVALID, "context is NULL");
  // work queued on either stream may still write into the caller's arena: let it finish before
  // the caller can free or reuse the arena (errors are reported but the context is still freed)
  const hipError_t e_main = hipStreamSynchronize(c->stream);
  const hipError_t e_side = c->side ? hipStreamSynchronize(c->side) : hipSuccess;
  for (hipEvent_t e : c->ev) hipEventDestroy(e);
  if (c->fork) hipEventDestroy(c->fork);
  if (c->join) hipEventDestroy(c->join);
  if (c->tail) hipEventDestroy(c->tail);
  if (c->wte_dw) hipEventDestroy(c->wte_dw);
  for (auto* v : {&c->ev_ln, &c->ev_dbig, &c->ev_dqkv, &c->ev_adam})
    for (hipEvent_t e : *v)
      if (e) hipEventDestroy(e);
  if (c->side) hipStreamDestroy(c->side);
  delete c;
  if (e_main != hipSuccess || e_side != hipSuccess)
    return fail(GPT2_E_HIP, std::string("stream synchronisation before destroy failed: ") +
                                hipGetErrorString(e_main != hipSuccess ? e_main : e_side));
  return GPT2_OK;
}

gpt2_status gpt2_join(gpt2_ctx* c) {
  STEP(check_ctx(c));
  HIPCHK(hipEventRecord(c->tail, c->side));
  HIPCHK(hipStreamWaitEvent(c->stream, c->tail, 0));
  return GPT2_OK;
}

static gpt2_status copy_flat(gpt2_ctx* c, int32_t set, float* dev, float* host, size_t n) {
  if (!host) return fail(GPT2_E_INVALID, "host buffer is NULL");
  if (n != (size_t)c->g.N) return fail(GPT2_E_INVALID, "n must equal the parameter count");
  HIPCHK(hipStreamSynchronize(c->stream));
  HIPCHK(hipStreamSynchronize(c->side));  // an AdamW update may still be running there
  if (set)
    HIPCHK(hipMemcpy(dev, host, n * sizeof(float), hipMemcpyHostToDevice));
  else
    HIPCHK(hipMemcpy(host, dev, n * sizeof(float), hipMemcpyDeviceToHost));
  return GPT2_OK;
}

gpt2_status gpt2_copy_params(gpt2_ctx* c, int32_t set, float* host, size_t n) {
  STEP(check_ctx(c));
  STEP(copy_flat(c, set, c->b.params, host, n));
  if (set && c->g.bf16) {
    HIPCHK(launch_cast_bf16(c->g.N, c->b.params, c->b.shadow, c->stream));
    HIPCHK(hipStreamSynchronize(c->stream));
  }
  return GPT2_OK;
}

gpt2_status gpt2_copy_grads(gpt2_ctx* c, int32_t set, float* host, size_t n) {
  STEP(check_ctx(c));
  return copy_flat(c, set, c->b.grads, host, n);
}

gpt2_status gpt2_copy_adam_state(gpt2_ctx* c, int32_t set, float* host_m, float* host_v, size_t n,
                                 int64_t* host_t) {
  STEP(check_ctx(c));
  if (!host_t) return fail(GPT2_E_INVALID, "t is NULL");
  STEP(copy_flat(c, set, c->b.m, host_m, n));
  STEP(copy_flat(c, set, c->b.v, host_v, n));
  if (set) {
    if (*host_t < 0) return fail(GPT2_E_INVALID, "t must be >= 0");
    c->t = *host_t;
  } else {
    *host_t = c->t;
  }
  return GPT2_OK;
}

gpt2_status gpt2_copy_row_loss(gpt2_ctx* c, float* host, size_t n) {
  STEP(check_ctx(c));
  if (!host) return fail(GPT2_E_INVALID, "host buffer is NULL");
  if (n != (size_t)c->g.M) return fail(GPT2_E_INVALID, "n must equal batch * seq_len");
  if (!c->have_forward) return fail(GPT2_E_STATE, "no forward has run");
  HIPCHK(hipStreamSynchronize(c->stream));
  HIPCHK(hipMemcpy(host, c->b.row_loss, n * sizeof(float), hipMemcpyDeviceToHost));
  return GPT2_OK;
}

gpt2_status gpt2_timing_begin(gpt2_ctx* c, int32_t family) {
  STEP(check_ctx(c));
  if (family < 0 || family >= FAM_COUNT)
    return fail(GPT2_E_INVALID, "family must be 0.." + std::to_string(FAM_COUNT - 1));
  if (c->ev.empty()) {
    c->ev.resize(2 * TIMING_CAP);
    for (auto& e : c->ev) HIPCHK(hipEventCreate(&e));
  }
  c->timing_family = family;
  c->timed = 0;
  c->timed_work = 0.0;
  return GPT2_OK;
}

gpt2_status gpt2_timing_end(gpt2_ctx* c, double* total_ms, int64_t* launches, double* work) {
  STEP(check_ctx(c));
  if (!total_ms || !launches || !work) return fail(GPT2_E_INVALID, "output pointer is NULL");
  c->timing_family = -1;
  HIPCHK(hipStreamSynchronize(c->stream));
  HIPCHK(hipStreamSynchronize(c->side));
  double ms = 0.0;
  for (int i = 0; i < c->timed; ++i) {
    float e = 0.0f;
    HIPCHK(hipEventElapsedTime(&e, c->ev[2 * i], c->ev[2 * i + 1]));
    ms += e;
  }
  *total_ms = ms;
  *launches = c->timed;
  *work = c->timed_work;
  return GPT2_OK;
}

gpt2_status gpt2_op_gemm(int32_t precision, int32_t a_kmajor, int32_t b_kmajor, int32_t m,
                         int32_t n, int32_t k, const void* d_a, int64_t lda, const void* d_b,
                         int64_t ldb, float* d_c, int64_t ldc, float alpha, float beta,
                         void* hip_stream) {
  if (precision != GPT2_FP32 && precision != GPT2_BF16) return fail(GPT2_E_INVALID, "precision");
  if (m < 0 || n < 0 || k < 0) return fail(GPT2_E_INVALID, "negative size");
  if (!d_a || !d_b || !d_c) return fail(GPT2_E_INVALID, "NULL operand");
  const int a_row = a_kmajor ? k : m, b_row = b_kmajor ? k : n;
  if (lda < a_row || ldb < b_row || ldc < n) return fail(GPT2_E_INVALID, "leading dimension too small");
  if (a_row % 8 || b_row % 8 || lda % 8 || ldb % 8)
    return fail(GPT2_E_UNSUPPORTED, "stored row lengths and leading dimensions must be multiples of 8");
  GemmParams p{};
  p.A = d_a; p.lda = lda; p.B = d_b; p.ldb = ldb; p.M = m; p.N = n; p.K = k; p.k_split = k;
  p.epi = EPI_F32; p.C = d_c; p.ldc = ldc; p.alpha = alpha; p.beta = beta;
  const bool bf = precision == GPT2_BF16;
  const int tile = bf ? gemm_pick_tile(m, n) : TILE_128;
  HIPCHK(launch_gemm(bf, a_kmajor ? 1 : 0, b_kmajor ? 1 : 0, tile, 1, 0, p,
                     static_cast<hipStream_t>(hip_stream)));
  return GPT2_OK;
}

static_assert(GPT2_EPI_STORE == EPI_STORE && GPT2_EPI_BIAS_GELU == EPI_BIAS_GELU &&
                  GPT2_EPI_BIAS_RESID == EPI_BIAS_RESID && GPT2_EPI_GELU_BWD == EPI_GELU_BWD,
              "ABI epilogue codes");

gpt2_status gpt2_op_gemm_epilogue(int32_t a_kmajor, int32_t b_kmajor, int32_t m, int32_t n,
                                  int32_t k, const void* d_a, int64_t lda, const void* d_b,
                                  int64_t ldb, int32_t epilogue, void* d_c, void* d_c2,
                                  int64_t ldc, const float* d_bias, const void* d_aux, float alpha,
                                  void* hip_stream) {
  if (m < 0 || n < 0 || k < 0) return fail(GPT2_E_INVALID, "negative size");
  if (epilogue < GPT2_EPI_STORE || epilogue > GPT2_EPI_GELU_BWD) return fail(GPT2_E_INVALID, "epilogue");
  const bool needs_c2 = epilogue == GPT2_EPI_BIAS_GELU;
  const bool needs_aux = epilogue == GPT2_EPI_BIAS_RESID || epilogue == GPT2_EPI_GELU_BWD;
  if (!d_a || !d_b || !d_c || (needs_c2 && !d_c2) || (needs_aux && !d_aux))
    return fail(GPT2_E_INVALID, "NULL operand");
  const int a_row = a_kmajor ? k : m, b_row = b_kmajor ? k : n;
  if (lda < a_row || ldb < b_row || ldc < n) return fail(GPT2_E_INVALID, "leading dimension too small");
  if (a_row % 8 || b_row % 8 || lda % 8 || ldb % 8 || n % 8 || ldc % 8)
    return fail(GPT2_E_UNSUPPORTED, "row lengths, n and leading dimensions must be multiples of 8");
  const void* ptrs[] = {d_a, d_b, d_c, d_c2, d_bias, d_aux};
  for (const void* q : ptrs)
    if (reinterpret_cast<uintptr_t>(q) % 16) return fail(GPT2_E_UNSUPPORTED, "pointers must be 16-byte aligned");
  GemmParams p{};
  p.A = d_a; p.lda = lda; p.B = d_b; p.ldb = ldb; p.M = m; p.N = n; p.K = k; p.k_split = k;
  p.epi = epilogue;  // the internal codes of these four epilogues are the ABI's
  p.C = d_c; p.C2 = d_c2; p.ldc = ldc; p.bias = epilogue == GPT2_EPI_GELU_BWD ? nullptr : d_bias;
  p.resid = epilogue == GPT2_EPI_BIAS_RESID ? static_cast<const float*>(d_aux) : nullptr;
  p.aux = epilogue == GPT2_EPI_GELU_BWD ? d_aux : nullptr;
  p.alpha = epilogue == GPT2_EPI_STORE ? alpha : 1.0f;
  p.beta = 0.0f;
  const int tile = gemm_pick_tile_epi(m, n, a_kmajor ? 1 : 0, b_kmajor ? 1 : 0, epilogue, false);
  HIPCHK(launch_gemm(true, a_kmajor ? 1 : 0, b_kmajor ? 1 : 0, tile, 1, 0, p,
                     static_cast<hipStream_t>(hip_stream)));
  return GPT2_OK;
}

static gpt2_status attn_args(int32_t precision, int32_t batch, int32_t seq_len, int32_t n_head,
                             int32_t head_dim) {
  if (precision != GPT2_FP32 && precision != GPT2_BF16) return fail(GPT2_E_INVALID, "precision");
  if (batch < 0 || seq_len < 0 || n_head < 1) return fail(GPT2_E_INVALID, "bad sizes");
  if (head_dim != 16 && head_dim != 32 && head_dim != 64)
    return fail(GPT2_E_UNSUPPORTED, "head_dim must be 16, 32 or 64");
  return GPT2_OK;
}

gpt2_status gpt2_op_attention_forward(int32_t precision, int32_t batch, int32_t seq_len,
                                      int32_t n_head, int32_t head_dim, const void* d_qkv,
                                      void* d_out, float* d_lse, void* hip_stream) {
  STEP(attn_args(precision, batch, seq_len, n_head, head_dim));
  if (!d_qkv || !d_out || !d_lse) return fail(GPT2_E_INVALID, "NULL buffer");
  HIPCHK(launch_attn_fwd(precision == GPT2_BF16, batch, seq_len, n_head, head_dim, d_qkv, d_out,
                         d_lse, static_cast<hipStream_t>(hip_stream)));
  return GPT2_OK;
}

gpt2_status gpt2_op_attention_backward(int32_t precision, int32_t batch, int32_t seq_len,
                                       int32_t n_head, int32_t head_dim, const void* d_qkv,
                                       const void* d_out, const float* d_lse, const void* d_dout,
                                       void* d_dqkv, float* d_scratch, void* hip_stream) {
  STEP(attn_args(precision, batch, seq_len, n_head, head_dim));
  if (!d_qkv || !d_out || !d_lse || !d_dout || !d_dqkv || !d_scratch)
    return fail(GPT2_E_INVALID, "NULL buffer");
  HIPCHK(launch_attn_bwd(precision == GPT2_BF16, batch, seq_len, n_head, head_dim, d_qkv, d_out,
                         d_lse, d_dout, d_dqkv, d_scratch, static_cast<hipStream_t>(hip_stream)));
  return GPT2_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- attention backward, no alloc
// The workspace of gpt2_op_attention_backward_noalloc: the attention backward's per-row pairs
// {log-sum-exp, D = rowsum(dO o O)} (2 floats per (batch, head, position)), written by its first
// kernel and read by its second within one call, so nothing in it has to start at zero. Each GPU
// the library runs on holds its own copy until the process ends. Host code never uses the
// array's name as an address (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, looked up once per device with that device current.
namespace {
constexpr int64_t NOALLOC_ATTN_FLOATS = int64_t(1) << 20;  // 4 MiB: batch*n_head*seq_len <= 2^19
static __device__ __align__(256) float scratch[NOALLOC_ATTN_FLOATS];

std::mutex g_scratch_mu;
std::vector<float*> g_scratch_dev;  // device address of `scratch`, per device id

gpt2_status scratch_for_stream(hipStream_t st, float** out) {
  int cur = 0;
  HIPCHK(hipGetDevice(&cur));
  int dev = cur;
  if (st) HIPCHK(hipStreamGetDevice(st, &dev));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_dev.size() <= dev) g_scratch_dev.resize(dev + 1, nullptr);
  if (!g_scratch_dev[dev]) {
    if (dev != cur) HIPCHK(hipSetDevice(dev));
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) HIPCHK(hipSetDevice(cur));
    if (e != hipSuccess)
      return fail(GPT2_E_HIP, std::string("hipGetSymbolAddress(scratch) failed: ") +
                                  hipGetErrorString(e));
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return GPT2_OK;
}
}  // namespace

extern "C" {

gpt2_status gpt2_op_attention_backward_noalloc(int32_t precision, int32_t batch, int32_t seq_len,
                                               int32_t n_head, int32_t head_dim,
                                               const void* d_qkv, const void* d_out,
                                               const float* d_lse, const void* d_dout,
                                               void* d_dqkv, void* hip_stream) {
  STEP(attn_args(precision, batch, seq_len, n_head, head_dim));
  if (!d_qkv || !d_out || !d_lse || !d_dout || !d_dqkv) return fail(GPT2_E_INVALID, "NULL buffer");
  const int64_t need = 2 * (int64_t)batch * n_head * seq_len;
  if (need > NOALLOC_ATTN_FLOATS)
    return fail(GPT2_E_UNSUPPORTED,
                "gpt2_op_attention_backward_noalloc: 2*batch*n_head*seq_len = " +
                    std::to_string(need) + " floats of scratch exceed its fixed " +
                    std::to_string(NOALLOC_ATTN_FLOATS) +
                    "; use gpt2_op_attention_backward with a workspace");
  const hipStream_t st = static_cast<hipStream_t>(hip_stream);
  float* ws = nullptr;
  STEP(scratch_for_stream(st, &ws));
  HIPCHK(launch_attn_bwd(precision == GPT2_BF16, batch, seq_len, n_head, head_dim, d_qkv, d_out,
                         d_lse, d_dout, d_dqkv, ws, st));
  return GPT2_OK;
}

}  // extern "C"
