/*
 * lss.h -- C ABI of the layer-skip self-speculative decoding engine (gfx950).
 *
 * The engine runs the draft -> verify -> accept -> layer-selection loop of
 * on-the-fly self-speculative greedy decoding for one sequence of a
 * Llama-style decoder on one GPU.  Sources of the method:
 *   - CLaSp article (news.43b.com.cn/a/479818), section 3 "workflow": draft
 *     with intermediate layers skipped, verify all drafts in one full-model
 *     pass, replace the first rejected draft with the full model's token and
 *     restart drafting there; choose the next skip set by a dynamic program
 *     over (i layers, j skipped) that maximizes cosine similarity to the last
 *     accepted token's full hidden states, all j of one i batched with a
 *     special attention mask instead of copied KV.
 *   - CAS-Spec summary page (arXiv 2510.26843), abstract, and the CAS-Spec
 *     blog (intelliparadigm.com 2260101), sections 2.1-3.2: draft models built
 *     from layer sparsity, early exit and dynamic 8-bit activation
 *     quantization; several draft levels routed by an EMA acceptance
 *     predictor (alpha = 0.2) and a linear latency model.
 *
 * Conventions for every entry point:
 *   - Return 0 on success or a negative lss_status.  On an argument or state
 *     error nothing is launched and the engine's committed state (length,
 *     window, skip bits, pending token) is unchanged.  lss_last_error()
 *     gives a message for the last failure of that engine.
 *   - Pointers named *_dev are device pointers; everything else is host
 *     memory owned by the caller and only read/written during the call.
 *   - All device work is enqueued on the stream given to lss_create.  Calls
 *     that return host values (tokens, counts) synchronize that stream.
 *   - One engine is not thread-safe; separate engines are independent.
 */
#ifndef LSS_H
#define LSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum lss_status {
  LSS_OK = 0,
  LSS_EINVAL = -1,     /* bad argument (sizes, null pointers, ranges) */
  LSS_ESTATE = -2,     /* call out of order (e.g. accept without verify) */
  LSS_ECAPACITY = -3,  /* KV capacity, window or row-block limit exceeded */
  LSS_EHIP = -4,       /* a HIP runtime call failed; see lss_last_error */
  LSS_ENOTIMPL = -5
};

enum lss_dtype { LSS_F32 = 0, LSS_BF16 = 1 };

/* Largest number of draft tokens a window can hold. */
#define LSS_WINDOW_MAX 31
/* Largest row block of one forward (verify rows, DP rows, prefill chunk). */
#define LSS_ROWS_MAX 64

/* Model and capacity description.  Weights use `dtype`, the KV cache
 * `kv_dtype`; activations and the residual stream are float32.  head_dim must be 64 or
 * 128; n_heads a multiple of n_kv_heads; d_model and ffn_dim multiples of
 * 32 (bf16) or 16 (float32), vocab a multiple of 16; d_model <= 8192. */
typedef struct lss_config {
  int32_t n_layers, d_model, n_heads, n_kv_heads, head_dim, ffn_dim, vocab;
  float rope_theta; /* rotary base; pairs (i, i + head_dim/2) */
  float rms_eps;    /* RMSNorm epsilon */
  int32_t dtype;    /* lss_dtype */
  int32_t max_seq;  /* KV capacity in positions (prompt + generated + window), <= 4096 */
  int32_t max_rows; /* row-block limit, 1..LSS_ROWS_MAX */
  int32_t kv_dtype; /* lss_dtype of the KV cache (float32 keeps keys/values unrounded) */
  int32_t max_seqs; /* independent sequences the engine holds, 0 or 1 (one) .. LSS_SEQS_MAX; each has
                       its own KV cache of max_seq positions (see lss_seq_select) */
} lss_config;

/* Largest number of sequences an engine holds, and of sequences one batched
 * pass takes (more go to further passes). */
#define LSS_SEQS_MAX 64
#define LSS_BATCH_PASS_SEQS 16

typedef struct lss_engine lss_engine;

/* Bytes of device workspace an engine needs for `cfg` (KV cache, residual
 * stash, activations, partial results).  0 if cfg is invalid. */
size_t lss_workspace_bytes(const lss_config* cfg);

/* One weight tensor handed to lss_load_weights (borrowed, never copied). */
typedef struct lss_tensor {
  const char* name;     /* canonical name, see lss_load_weights */
  const void* dev_ptr;  /* device pointer, 16-byte aligned */
  int64_t numel;        /* element count, checked against the config */
} lss_tensor;

/* load_weights: create an engine over an existing model's weights (the
 * method is plug-and-play over a trained model, no training step: CLaSp
 * article, introduction and section 3; CAS-Spec abstract).
 * tensors: n_tensors = 3 + 9*n_layers entries in the canonical order
 *   "embed" [V][d], "final_norm" [d], "lm_head" [V][d], then for each layer
 *   l: "layers.<l>.attn_norm" [d], ".wq" [Hq*hd][d], ".wk" [Hkv*hd][d],
 *   ".wv" [Hkv*hd][d], ".wo" [d][Hq*hd], ".ffn_norm" [d], ".w_gate" [F][d],
 *   ".w_up" [F][d], ".w_down" [d][F]; matrices row-major [out][in] in
 *   cfg->dtype, norm gains float32.  A wrong name, element count, null or
 *   misaligned pointer is LSS_EINVAL.
 * workspace_dev: >= lss_workspace_bytes(cfg) bytes of device memory, 256-byte
 *   aligned (LSS_ECAPACITY if smaller).
 * Weights and workspace are borrowed (never freed) and must outlive the
 * engine; the engine allocates only two small pinned host buffers of its
 * own.  hip_stream: a hipStream_t (NULL = the null stream); every later
 * call of the engine enqueues its device work there.  On failure *out is
 * NULL and lss_last_error(NULL) describes the failure (per thread). */
int lss_load_weights(const lss_config* cfg, const lss_tensor* tensors, int32_t n_tensors,
                     void* workspace_dev, size_t workspace_bytes, void* hip_stream, lss_engine** out);
/* The same with bare pointers in the canonical order (no name or size
 * check). */
int lss_create(const lss_config* cfg, const void* const* tensors_dev, int32_t n_tensors,
               void* workspace_dev, size_t workspace_bytes, void* hip_stream, lss_engine** out);
void lss_destroy(lss_engine* e);
/* Message of the engine's last failure; with e == NULL, of this thread's
 * last failed lss_load_weights / lss_create or stand-alone acceptance op. */
const char* lss_last_error(const lss_engine* e);

/* Full-model causal pass over the prompt (row blocks of max_rows).  Resets
 * the sequence.  *t0_out = greedy next token (with sampling on: the full
 * model's draw at the last prompt row), which becomes the pending token; the
 * last prompt row becomes the layer-selection target. */
int lss_prefill(lss_engine* e, const int32_t* tokens, int32_t n, int32_t* t0_out);

/* Speculative sampling (the pages call the scheme lossless: it keeps the
 * full model's output distribution -- CAS-Spec abstract; CLaSp section 3,
 * verification predicts a distribution per draft token; CLaSp section 4).
 * temperature > 0 turns it on for the following calls, 0 returns to greedy
 * decoding.  Every random draw is a pure function of (seed, purpose,
 * position, index): Philox-4x64-10 with key (seed, purpose) and counter
 * (index / 4, position, 0, 0), word index % 4, uniform
 * ((x >> 41) + 1/2) / 2^23, Gumbel noise -log(-log u); purposes 1 draft
 * draw, 2 full-model draw, 3 acceptance uniform, 4 replacement draw; the
 * position is that of the row whose distribution is drawn from or tested.
 *   - draws: argmax of z / T + Gumbel noise (a draw from softmax(z / T));
 *   - draft i is accepted iff r q(d) < p(d) (p, q at temperature T; r the
 *     acceptance uniform of verify row i's position);
 *   - the first rejection draws the replacement from max(0, p - q)
 *     (Gumbel-max over log of it; from p if rounding leaves it empty);
 *     with every draft accepted the bonus is the draw of verify row k;
 *   - the draft exit threshold compares the top-1 probability at T.
 * LSS_EINVAL for a negative or non-finite temperature; LSS_ESTATE while a
 * draft window or verify is pending.  Host-forced drafts (lss_verify with
 * drafts != NULL and k > 0) are rejected with LSS_EINVAL in this mode: they
 * carry no draft distribution. */
int lss_set_sampling(lss_engine* e, float temperature, uint64_t seed);

/* Draft up to k tokens with the layers where skip_mask[l] != 0 skipped
 * (CLaSp section 3, draft stage; an early exit is a mask whose tail is
 * skipped).  quant = 1 quantizes every projection input of an executed
 * layer to int8 per token (CAS-Spec blog section 2.1); quant = 2 also
 * replaces that layer's weights by their int8 copy (lss_attach_w8: the
 * 8-bit strategy carried over to the weights, the bytes a batch-1 draft
 * streams halved; LSS_ESTATE if no copy is attached).  exit_tau > 0 stops
 * after the first token whose top-1 softmax probability is below exit_tau
 * (CLaSp section 4, draft exit threshold).  Appends to the pending window
 * (several levels may draft into one window).  tokens_out[k] receives the
 * drafted tokens, *k_done their count.  LSS_ECAPACITY if the window would
 * exceed LSS_WINDOW_MAX or max_rows - 1 tokens or the KV capacity. */
int lss_draft(lss_engine* e, const uint8_t* skip_mask, int32_t quant, int32_t k, float exit_tau,
              int32_t* tokens_out, int32_t* k_done);

/* Token-tree draft of width B (1 <= B <= 8) and depth D >= 1, the pages'
 * "dynamic tree cascade" read as a token tree (CAS-Spec abstract; CAS-Spec
 * blog section 3): the draft (skip mask, quant as in lss_draft) runs the
 * pending token's row at position p and takes its B most likely tokens
 * (largest logit first, ties to the lower id) as the first nodes of B
 * branches for position p + 1, then extends every branch greedily by D - 1
 * tokens, all branches' rows of one depth in one draft pass (node j of a
 * branch, at position p + j, sees the committed prefix, the pending token
 * and its branch's nodes 1..j only).  tokens_out[B * D] receives the
 * branches one after the other (branch b's node j at index b D + j - 1).
 * lss_verify(e, NULL, B * D) then verifies every node in one pass with a
 * tree mask (each node's row equals the full model's step after its
 * branch's earlier nodes, bit for bit) and accepts greedily: the branch
 * whose first node equals the full model's token after the pending one is
 * followed while each next node equals the full model's token after the
 * previous one; n = accepted nodes, the bonus the full model's token after
 * the last of them (n = 0 and that first token when no branch matches);
 * the accepted nodes' keys and values become positions p + 1 .. p + n.
 * Greedy only (LSS_EINVAL with sampling on); LSS_ESTATE unless the window
 * is empty; LSS_ECAPACITY if B D > LSS_TREE_NODES_MAX, B D + 1 > max_rows
 * or the KV capacity is exceeded. */
#define LSS_TREE_NODES_MAX 15
int lss_draft_tree(lss_engine* e, const uint8_t* skip_mask, int32_t quant, int32_t B, int32_t D, int32_t* tokens_out);

/* The same tree with a draft level per depth: the cascade's levels routed
 * into the tree (CAS-Spec abstract, dynamic tree cascade; CAS-Spec blog
 * section 2.2, levels).  The nodes of depth j (1 .. D) come from the pass
 * with skip mask masks[(j - 1) * n_layers ..] (1 = skip) and quant
 * quants[j - 1] (0, 1 or 2 as in lss_draft): the pending token's row for
 * j = 1, the rows of the depth j - 1 nodes otherwise.  In a layer, a row
 * sees the pending token and its branch's node i only where the pass over
 * them ran that layer (per-layer valid bits by depth, as in a chain window
 * drafted by several levels).  lss_draft_tree is this call with one level
 * at every depth.  masks and quants are host arrays of the caller, read
 * during the call.  Errors as lss_draft_tree, plus LSS_EINVAL for a quant
 * outside 0..2 and LSS_ESTATE for quant 2 without lss_attach_w8. */
int lss_draft_tree_levels(lss_engine* e, const uint8_t* masks, const int32_t* quants, int32_t B, int32_t D,
                          int32_t* tokens_out);

/* Verify the window in one full-model pass over rows [t0, d1..dk] at
 * positions p..p+k (CLaSp section 3, verification).  drafts == NULL
 * verifies the pending window; otherwise the k host tokens replace it (a
 * host-forced draft).  Acceptance is computed on the device; results are
 * read by lss_accept_and_rollback. */
int lss_verify(lss_engine* e, const int32_t* drafts, int32_t k);

/* Greedy acceptance and O(1) rollback: n = longest prefix of the drafts that
 * equals the full model's argmax tokens, bonus = the full model's token
 * after it (with sampling on: n and the bonus come from the speculative-
 * sampling rule of lss_set_sampling, decided on the device in verify).  The committed length becomes p + n + 1 (later KV rows are stale
 * and never read), the window is cleared, the bonus token is pending, and
 * verify row n becomes the layer-selection target.  accepted_out (may be
 * NULL) receives the n + 1 emitted tokens d1..dn, bonus. */
int lss_accept_and_rollback(lss_engine* e, int32_t* n_accepted, int32_t* bonus,
                            int32_t* accepted_out);

/* CLaSp layer selection (section 3): skip exactly n_skip of the n_layers
 * layers by the batched cosine-similarity DP against the target's full
 * hidden states (the last accepted token's; after prefill, the last prompt
 * row's).  mask_out[n_layers] gets 1 = skip; score_out (may be NULL) the
 * final cosine similarity.  LSS_EINVAL unless 0 <= n_skip <= n_layers. */
int lss_select_layers_dp(lss_engine* e, int32_t n_skip, uint8_t* mask_out, float* score_out);
/* The same DP over the first n_layers_eff layers only (n_layers_eff <=
 * n_layers): the layers past it are marked skipped, an early exit (the
 * CAS-Spec blog's draft levels with layer sparsity plus early exit,
 * section 2.2). */
int lss_select_layers_dp_exit(lss_engine* e, int32_t n_skip, int32_t n_layers_eff, uint8_t* mask_out,
                              float* score_out);

/* Committed sequence length p. */
int32_t lss_seq_len(const lss_engine* e);

/* ---- Several sequences (batch > 1).  Neither page batches requests; a
 * batch here is a set of independent sequences, each decoded exactly as on
 * its own (the same drafts, acceptances and tokens; CLaSp article, section
 * 3, per sequence), whose rows share passes over the weights.
 *
 * lss_seq_select: sequence `seq` (0 .. max_seqs - 1) becomes the current
 * one; every single-sequence call (prefill, draft, draft_tree, verify,
 * accept_and_rollback, select_layers_dp, generate, seq_len) acts on it and
 * on its own KV cache, window, layer-selection target and results.
 * LSS_EINVAL for a bad index; LSS_ESTATE when sampling is on and the
 * current sequence has an unverified window (its draft distributions share
 * one buffer).  The logits and residual-state readers return the engine's
 * last pass, whichever sequence(s) it served. */
int lss_seq_select(lss_engine* e, int32_t seq);

/* Batched draft of n distinct sequences seqs[n] (each prefilled, no verify
 * pending, no tree window): sequence seqs[i] appends up to k[i] tokens to
 * its window with its own skip mask masks[i * n_layers ..] (1 = skip),
 * stopping early when its draft's top-1 probability falls below exit_tau
 * (> 0), exactly as lss_draft would.  Sequences with identical masks share
 * each draft step's pass (one row each, at their own positions).  quant: 0
 * or 1 (int8 activations); the W8A8 draft (2) is single-row only
 * (LSS_EINVAL).  tokens_out[i * LSS_WINDOW_MAX + j] receives sequence i's
 * j-th new token, k_done[i] their count.  Greedy only (LSS_EINVAL with
 * sampling on).  LSS_ECAPACITY as lss_draft, per sequence; nothing is
 * drafted then. */
int lss_batch_draft(lss_engine* e, int32_t n, const int32_t* seqs, const uint8_t* masks, int32_t quant,
                    const int32_t* k, float exit_tau, int32_t* tokens_out, int32_t* k_done);

/* Batched verify of the pending windows of n distinct sequences (a window
 * may be empty: a greedy step).  Each sequence's rows [pending token,
 * drafts] at its own positions see only its own cache, causally; every row
 * equals the single-sequence verify row bit for bit.  Sequences are packed
 * into passes of at most max_rows rows and LSS_BATCH_PASS_SEQS sequences.
 * Acceptance runs on the device per sequence; lss_batch_accept reads it. */
int lss_batch_verify(lss_engine* e, int32_t n, const int32_t* seqs);

/* Accept and roll back each listed sequence after lss_batch_verify, as
 * lss_accept_and_rollback: n_accepted[i], bonus[i], and
 * accepted_out[i * (LSS_WINDOW_MAX + 1) ..] the n_accepted[i] + 1 emitted
 * tokens (any output may be NULL). */
int lss_batch_accept(lss_engine* e, int32_t n, const int32_t* seqs, int32_t* n_accepted, int32_t* bonus,
                     int32_t* accepted_out);

/* Parity helpers: logits [rows][vocab] of the last verify / draft step /
 * prefill row; residual states [n_layers + 1][d] of verify row `row` (valid
 * until the next draft, verify or prefill); the last DP's decisions
 * [n_layers + 1][n_layers + 1] (stage i, skipped count j) as float triples
 * {skip chosen, cos(skip candidate), cos(executed candidate)}, NaN where a
 * state or candidate does not exist. */
int lss_read_logits(lss_engine* e, int32_t rows, float* host_out);
int lss_read_states(lss_engine* e, int32_t row, float* host_out);
int lss_read_dp_decisions(lss_engine* e, float* host_out);

/* Draft policy of lss_generate. */
enum lss_mode { LSS_MODE_AR = 0, LSS_MODE_STATIC = 1, LSS_MODE_DP = 2, LSS_MODE_CASCADE = 3 };
#define LSS_LEVELS_MAX 4
#define LSS_STOP_MAX 8
typedef struct lss_policy {
  int32_t mode;              /* lss_mode */
  int32_t k_max;             /* draft tokens per round (cascade: total) */
  float exit_tau;            /* draft exit threshold, <= 0 off */
  int32_t quant;             /* STATIC / DP drafts: int8 activations */
  const uint8_t* static_mask;/* STATIC: [n_layers] 1 = skip */
  int32_t n_skip;            /* DP: layers to skip */
  int32_t interval;          /* DP / CASCADE: re-run the DP every `interval` verify rounds */
  int32_t n_levels;          /* CASCADE: levels, index 0 = fastest */
  int32_t level_skip[LSS_LEVELS_MAX];  /* total skipped layers per level (incl. exit tail) */
  int32_t level_exit[LSS_LEVELS_MAX];  /* early-exit tail length per level */
  int32_t level_quant[LSS_LEVELS_MAX]; /* int8 activations per level */
  double beta[3];            /* CASCADE latency model b0 + b1*seq_len + b2*executed_layers */
  int32_t tree_width;        /* STATIC / DP: > 0 drafts a width-B token tree per round (lss_draft_tree);
                                CASCADE: > 0 routes the levels into a tree per round, width <= tree_width
                                chosen by lss_router_plan_tree (lss_draft_tree_levels) */
  int32_t tree_depth;        /* STATIC / DP tree depth (0 or 1: depth 1), cut to the tokens still to emit */
  double row_cost[LSS_TREE_NODES_MAX + 1]; /* CASCADE trees: cost factor of a pass over r rows at index
                                r - 1 (all 0: 1 for every row count) */
  int32_t n_stop;            /* stop tokens (0: none, at most LSS_STOP_MAX): generation ends right after the
                                first emitted token that is one of stop_tokens[0 .. n_stop) */
  int32_t stop_tokens[LSS_STOP_MAX];
} lss_policy;

typedef struct lss_stats {
  int32_t rounds, drafted, accepted, dp_runs, emitted;
} lss_stats;

/* Prefill `prompt`, then decode until n_gen tokens (t0 included) are
 * emitted into out_tokens[n_gen] with the given policy; LSS_MODE_AR is the
 * greedy autoregressive baseline (verify of the pending token alone).  With
 * stop tokens, decoding ends early right after the first emitted stop token
 * (which is kept); stats->emitted is the number of tokens written.  Those
 * tokens are the first ones of the run without stop tokens, so the output
 * stays lossless.  The engine's committed sequence may then hold the rest
 * of that round's accepted tokens.  LSS_EINVAL for n_stop outside
 * [0, LSS_STOP_MAX] or a stop token outside the vocabulary. */
int lss_generate(lss_engine* e, const int32_t* prompt, int32_t n_prompt, int32_t n_gen,
                 const lss_policy* policy, int32_t* out_tokens, lss_stats* stats);

/* Decode n_seqs prompts together (sequences 0 .. n_seqs - 1; prompt i is
 * prompt_lens[i] tokens at prompts + sum of the earlier lengths) until each
 * has n_gen tokens in out_tokens[i * n_gen ..]: every sequence runs the
 * policy's rounds as lss_generate would on its own (LSS_MODE_AR, STATIC, or
 * DP with its own layer selection), the rounds of all sequences batched.
 * stats[n_seqs] per sequence (may be NULL).  Stop tokens end each
 * sequence on its own as in lss_generate; a stopped sequence leaves the
 * batch, and the rest of its out_tokens row is left untouched.  The cascade
 * mode, trees, sampling and the W8A8 draft are single-sequence only
 * (LSS_EINVAL). */
int lss_generate_batch(lss_engine* e, int32_t n_seqs, const int32_t* prompts, const int32_t* prompt_lens,
                       int32_t n_gen, const lss_policy* policy, int32_t* out_tokens,
                       lss_stats* stats);

/* DyTC router on the host (CAS-Spec blog sections 3.1-3.2, CAS-Spec
 * abstract).  plan: draft length per level (index 0 = fastest) maximizing
 * (E + 1) / (t_verify + sum k_l t_hat_l), E the expected accepted length of
 * the window ordered most precise level first, total <= k_max.  update:
 * EMA (alpha 0.2) of each level's accepted/reached ratio after a round
 * whose window slots had levels slot_levels[k] and n were accepted.
 * fit: least squares b for samples [n][3] = {seq_len, depth, seconds}. */
int lss_router_plan(const double* accept_rate, const double* t_hat, int32_t n_levels,
                    double t_verify, int32_t k_max, int32_t* plan_out);
int lss_router_update(double* accept_rate, int32_t n_levels, const int32_t* slot_levels,
                      int32_t k, int32_t n_accepted);
/* Tree routing (the abstract's dynamic tree cascade; our reading): a width
 * B and draft lengths per level plan_out[n_levels] (index 0 = fastest) for
 * a token tree whose depths are drafted precise level first.  Expected
 * accepted nodes E = h (1 + sum_{j>=2} prod_{2<=m<=j} a_level(m)) with
 * h = 1 - (1 - a_level(1))^B (B independent first candidates); predicted
 * time = t_verify row_cost[B D] + the depth passes (the first over one row:
 * t_hat row_cost[0], later ones over B rows: t_hat row_cost[B - 1]);
 * row_cost NULL means 1.  Maximizes (E + 1) / time over 1 <= B <= b_max and
 * totals D <= k_max with B D <= nodes_max; ties: fewer nodes, smaller
 * width, then the order of lss_router_plan.  A total of 0 (width 1) is a
 * greedy step.  update_tree: EMA update after a tree round whose depths had
 * levels depth_levels[D] and n nodes accepted along branch `branch` (-1
 * when n = 0): the first depth counts as accepted only for branch 0 (the
 * draft's most likely token), later depths along the branch followed.
 * LSS_EINVAL for sizes out of range. */
int lss_router_plan_tree(const double* accept_rate, const double* t_hat, int32_t n_levels, double t_verify,
                         const double* row_cost, int32_t k_max, int32_t b_max, int32_t nodes_max,
                         int32_t* width_out, int32_t* plan_out);
int lss_router_update_tree(double* accept_rate, int32_t n_levels, const int32_t* depth_levels, int32_t D,
                           int32_t n_accepted, int32_t branch);
int lss_latency_fit(const double* samples, int32_t n, double* beta_out);

/* Measurement: time every launch of one GEMM family with HIP events on the
 * engine stream.  epilogue: 0 = fused q/k/v projection, 1 = projection +
 * residual add (attention output, FFN down), 2 = gate/up projection + SwiGLU,
 * 3 = LM head + argmax partials; 16 + the same code selects the int8 GEMV
 * of the W8A8 draft (16 q/k/v, 17 residual, 18 gate/up); rows: match only
 * launches with this many rows (0 = any).  enable = 0 stops recording.  lss_profile_read syncs the
 * stream and returns the summed launch time, the launch count and the summed
 * algorithmic bytes (weights + activation rows read + output rows written)
 * since profiling was enabled. */
int lss_profile_kernel(lss_engine* e, int32_t epilogue, int32_t rows, int32_t enable);
int lss_profile_read(lss_engine* e, double* total_ms, int64_t* launches, int64_t* bytes);

/* Grid of the decode GEMV (the vector-ALU projection of draft, greedy and
 * verify rows): wgs_per_cu = 0 launches one workgroup per weight tile.
 * wgs_per_cu > 0 allows at most that many workgroups per compute unit
 * (capped by the kernel's occupancy): launches with more than 4 times that
 * many tiles then run that many workgroups, each walking a contiguous range
 * of tiles with its weight loads kept in flight across tile boundaries;
 * smaller launches keep one workgroup per tile.  The arithmetic of every
 * output is the same under any grid, so results are identical bit for bit;
 * only the time changes.  The default is 1.  LSS_EINVAL for a negative
 * value or a value above 8. */
int lss_set_gemv_grid(lss_engine* e, int32_t wgs_per_cu);

/* Kernel of the decode rows with bf16 weights (projections of draft steps,
 * verify passes and greedy steps):
 *   kind 0 (the default): the vector-ALU GEMV for every decode row -- the
 *     fastest at 1 or 2 rows; rows beyond its register budget (8 at
 *     K = 4096, 4 at K = 14336, 2 at K = 28672) go to further launches;
 *   kind 1: the MFMA GEMM for every decode row -- one launch that streams
 *     each weight byte once for up to 16 rows;
 *   kind 2: the MFMA GEMM for the full-model rows (verify, greedy steps),
 *     the vector-ALU GEMV for the draft rows.
 * Under every kind a verify row gets the bits of the greedy step at the
 * same position (both are full-model rows); with kinds 0 and 1 a draft that
 * skips nothing also equals the full model bit for bit.  The kinds differ
 * in rounding only.  Float32 weights always take the vector-ALU GEMV.
 * LSS_EINVAL for another kind, LSS_ESTATE while a draft window or verify is
 * pending. */
int lss_set_decode_kernel(lss_engine* e, int32_t kind);

/* Stand-alone dynamic per-token int8 quantization (CAS-Spec blog section
 * 2.1): for each of `rows` rows of x_dev[rows][n] (float32), codes q_dev
 * [rows][n] = clamp(rint(x * fl(127/amax)), -127, 127) and scale_dev[rows]
 * = amax/127, all in float32, amax = 0 giving codes 0 and scale 0.
 * Enqueued on hip_stream; no synchronization. */
int lss_op_quantize_rows(const float* x_dev, int32_t rows, int32_t n, int8_t* q_dev,
                         float* scale_dev, void* hip_stream);

/* Stand-alone greedy acceptance, the fused argmax-compare step of
 * verification (CLaSp article, section 3: the full model scores every draft
 * in one pass; the first draft that differs from the full model's token is
 * replaced by it and the rest are dropped) on logits the caller holds.
 *   logits_dev: [rows][vocab] float32, the verify rows [t0, d1..dk] (rows =
 *     k + 1, 1 <= rows <= LSS_ACCEPT_ROWS_MAX);
 *   drafts_dev: [rows - 1] int32 draft tokens d1..dk (may be NULL if rows
 *     is 1);
 *   result_dev: [2 + rows] int32, written on the device: result[0] = n, the
 *     length of the longest prefix of the drafts equal to the rows' argmax
 *     tokens (lowest index on ties; NaN never wins; a row of NaNs gives 0),
 *     result[1] = the bonus token (argmax of row n), result[2 + r] = argmax
 *     of row r.
 * lss_op_accept_greedy_workspace_bytes: scratch bytes the op needs (0 for
 * invalid sizes).  lss_op_accept_greedy takes that scratch as workspace_dev
 * (caller-owned device memory, 8-byte aligned; LSS_ECAPACITY if smaller).
 * Enqueued on hip_stream, no synchronization; LSS_EINVAL for bad sizes or
 * null pointers.  On failure lss_last_error(NULL) describes it. */
#define LSS_ACCEPT_ROWS_MAX 64
#define LSS_ACCEPT_VOCAB_MAX 262144
size_t lss_op_accept_greedy_workspace_bytes(int32_t rows, int32_t vocab);
int lss_op_accept_greedy(const float* logits_dev, int32_t rows, int32_t vocab, const int32_t* drafts_dev,
                         int32_t* result_dev, void* workspace_dev, size_t workspace_bytes, void* hip_stream);

/* The same with no workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): its scratch is a fixed 32 KB array inside the library,
 * one per GPU, held until the process ends; vocab <= LSS_ACCEPT_VOCAB_MAX
 * (LSS_ECAPACITY above it).  It calls no allocating routine.  All calls on
 * one GPU share that array: calls that overlap on one GPU (several streams,
 * several host threads) race and must be ordered by the caller. */
int lss_op_accept_greedy_noalloc(const float* logits_dev, int32_t rows, int32_t vocab, const int32_t* drafts_dev,
                                 int32_t* result_dev, void* hip_stream);

/* int8 weight copy for the W8A8 draft (lss_draft quant = 2): the 8-bit
 * dynamic quantization of CAS-Spec blog section 2.1 applied per output row
 * to the weights of every layer's seven projections.  Each row gets the
 * activation rule: codes clamp(rint(w * fl(127/amax)), -127, 127), scale
 * amax/127 (float32 decisions).  lss_w8_bytes: bytes the copy needs (0 for
 * an invalid config).  lss_attach_w8 quantizes the engine's weights into
 * the caller-owned device buffer (256-byte aligned, at least lss_w8_bytes;
 * it must outlive the engine), synchronously on the engine stream.
 * LSS_EINVAL for a null or unaligned buffer, LSS_ECAPACITY if too small. */
size_t lss_w8_bytes(const lss_config* cfg);
int lss_attach_w8(lss_engine* e, void* buf_dev, size_t bytes);

/* Stand-alone forms of the two W8A8 kernels, enqueued on hip_stream:
 * lss_op_w8_quantize: codes q_dev[rows][k] and scale_dev[rows] of a weight
 *   matrix w_dev[rows][k] of dtype LSS_F32 or LSS_BF16 (rule above);
 * lss_op_w8a8_gemv: one activation row of codes xq_dev[k] with scale
 *   xscale_dev[0] against wq_dev[n][k] with row scales wscale_dev[n]:
 *   y_dev[n] = fl32(fl32(acc) * fl32(wscale[n] * xscale)), acc the exact
 *   integer dot product;
 * lss_op_w8a8_gemv_f32: the same with a float32 row x_dev[k], quantized in
 *   the kernel by the per-token rule of lss_op_quantize_rows (the form the
 *   W8A8 draft runs: every workgroup forms the codes itself).
 * n and k multiples of 16, k <= 32768, wq_dev and xq_dev 16-byte aligned;
 * LSS_EINVAL otherwise. */
int lss_op_w8_quantize(const void* w_dev, int32_t dtype, int32_t rows, int32_t k, int8_t* q_dev,
                       float* scale_dev, void* hip_stream);
int lss_op_w8a8_gemv(const int8_t* wq_dev, const float* wscale_dev, int32_t n, int32_t k, const int8_t* xq_dev,
                     const float* xscale_dev, float* y_dev, void* hip_stream);
int lss_op_w8a8_gemv_f32(const int8_t* wq_dev, const float* wscale_dev, int32_t n, int32_t k, const float* x_dev,
                         float* y_dev, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* LSS_H */
