// Decode-step graphs: one HIP graph per batch bucket, each holding the step's
// KV store fused into paged decode attention (split pass + merge) on static
// buffers, for one layer or for every layer of the model in order: two
// kernels per layer.
//
// P1 = "13. 读一个最小推理引擎：nano-vllm", "第五站：执行准备与 KV 容量" (CUDA
// Graph paragraph): decode only, one graph per bucket (1, 2, 4, 8, then
// steps of 16), captured largest first; at run time the smallest bucket that
// holds the batch is replayed after the inputs are copied into its static
// buffers and the padding rows get slot -1. "其余部分" of the same page
// notes that graphs pay off for small-model decode, which is launch-bound.
//
// The graphs capture the library's own entry points, so replay computes
// exactly what the eager calls compute on the same buffers. A captured
// decode stays valid for any context lengths up to max_context_len: the
// decode kernels read the lengths on the device and derive their split of
// the work from them. No graph contains a memset or an allocation; the
// decode workspace needs no initialisation.

#include <new>
#include <vector>

#include "common.h"

struct pkv_decode_graphs {
  std::vector<pkv_decode_graph_desc> layers;  // one step = these descriptors' calls, in order
  std::vector<int32_t> buckets;       // ascending
  std::vector<hipGraphExec_t> execs;  // one per bucket
  std::vector<hipGraph_t> graphs;
  ~pkv_decode_graphs() {
    for (hipGraphExec_t e : execs)
      if (e) (void)hipGraphExecDestroy(e);
    for (hipGraph_t g : graphs)
      if (g) (void)hipGraphDestroy(g);
  }
};

namespace {

// the decode step (every layer's store + attention) on the first `rows` rows of the static buffers
pkv_status enqueue_step(const std::vector<pkv_decode_graph_desc>& layers, int32_t rows, hipStream_t s) {
  for (const pkv_decode_graph_desc& d : layers) {
    const pkv_status st = paged_attn_decode_store(
        d.out, d.q, d.key, d.key_stride, d.value, d.value_stride, d.slot_mapping, d.k_cache, d.v_cache,
        d.block_tables, d.block_table_stride, d.context_lens, rows, d.num_q_heads, d.num_kv_heads, d.head_dim,
        d.block_size, d.num_blocks, d.scale, d.max_context_len, d.workspace, d.workspace_bytes, s);
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

}  // namespace

extern "C" pkv_status pkv_decode_graphs_create(const pkv_decode_graph_desc* desc, const int32_t* buckets,
                                               int32_t num_buckets, pkv_decode_graphs** out) {
  return pkv_decode_graphs_create_layers(desc, 1, buckets, num_buckets, out);
}

extern "C" pkv_status pkv_decode_graphs_create_layers(const pkv_decode_graph_desc* layers, int32_t num_layers,
                                                      const int32_t* buckets, int32_t num_buckets,
                                                      pkv_decode_graphs** out) {
  using pkv::fail;
  if (!out) return fail(PKV_ERR_INVALID, "pkv_decode_graphs_create: null output");
  *out = nullptr;
  if (!layers || num_layers < 1) return fail(PKV_ERR_INVALID, "pkv_decode_graphs_create: no layers");
  if (!buckets || num_buckets < 1) return fail(PKV_ERR_INVALID, "pkv_decode_graphs_create: no buckets");
  for (int32_t i = 0; i < num_buckets; ++i)
    if (buckets[i] < 1 || (i && buckets[i] <= buckets[i - 1]))
      return fail(PKV_ERR_INVALID, "pkv_decode_graphs_create: buckets must be positive and ascending");
  // argument errors surface from the entry points while the first graph is
  // captured; the decode launch's device queries are made here, outside capture
  for (int32_t l = 0; l < num_layers; ++l)
    for (int32_t i = 0; i < num_buckets; ++i)
      if (!pkv::decode_prepare(layers[l].num_q_heads, layers[l].num_kv_heads, buckets[i])) break;
  pkv_decode_graphs* g = new (std::nothrow) pkv_decode_graphs;
  if (!g) return fail(PKV_ERR_INVALID, "pkv_decode_graphs_create: out of host memory");
  g->layers.assign(layers, layers + num_layers);
  g->buckets.assign(buckets, buckets + num_buckets);
  g->execs.assign(num_buckets, nullptr);
  g->graphs.assign(num_buckets, nullptr);
  hipStream_t cs = nullptr;
  if (hipStreamCreateWithFlags(&cs, hipStreamNonBlocking) != hipSuccess) {
    delete g;
    return fail(PKV_ERR_HIP, "pkv_decode_graphs_create: stream creation failed");
  }
  pkv_status result = PKV_OK;
  for (int32_t i = num_buckets - 1; i >= 0 && result == PKV_OK; --i) {  // largest first
    hipError_t e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
      result = fail(PKV_ERR_HIP, "pkv_decode_graphs_create: begin capture: %s", hipGetErrorString(e));
      break;
    }
    pkv_status st = enqueue_step(g->layers, g->buckets[i], cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    g->graphs[i] = graph;
    if (st != PKV_OK) {
      result = st;
      break;
    }
    if (e != hipSuccess || !graph) {
      result = fail(PKV_ERR_HIP, "pkv_decode_graphs_create: end capture: %s", hipGetErrorString(e));
      break;
    }
    e = hipGraphInstantiate(&g->execs[i], graph, nullptr, nullptr, 0);
    if (e != hipSuccess) result = fail(PKV_ERR_HIP, "pkv_decode_graphs_create: instantiate: %s", hipGetErrorString(e));
  }
  (void)hipStreamDestroy(cs);
  if (result != PKV_OK) {
    delete g;
    return result;
  }
  *out = g;
  return pkv::ok();
}

extern "C" pkv_status pkv_decode_graphs_launch(pkv_decode_graphs* g, int32_t batch, int32_t* out_bucket,
                                               void* stream) {
  using pkv::fail;
  if (!g) return fail(PKV_ERR_INVALID, "pkv_decode_graphs_launch: null handle");
  if (batch < 1 || batch > g->buckets.back())
    return fail(PKV_ERR_INVALID, "pkv_decode_graphs_launch: batch %d outside [1, %d]", batch, g->buckets.back());
  size_t i = 0;
  while (g->buckets[i] < batch) ++i;
  if (out_bucket) *out_bucket = g->buckets[i];
  const hipError_t e = hipGraphLaunch(g->execs[i], reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "pkv_decode_graphs_launch: %s", hipGetErrorString(e));
  return pkv::ok();
}

extern "C" pkv_status pkv_decode_graphs_destroy(pkv_decode_graphs* g) {
  delete g;
  return pkv::ok();
}
