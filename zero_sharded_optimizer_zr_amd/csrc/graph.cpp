// Captured steps: a sequence of library calls recorded once on a stream as a
// HIP graph and replayed as one launch.  Small shards are launch-bound (the
// tiny MLP's four-call step moves 14 MB in 40 us of launches), and a training
// loop repeats the same calls on the same buffers every step; what changes is
// the AdamW step number t (its bias corrections) and possibly the learning
// rate.  Those enter the AdamW-family kernels as one by-value argument
// (AdamWScalars), so the graph keeps, for every captured kernel node that
// takes it, the node and its argument list, and zr_graph_set_adamw rewrites
// that one argument on the instantiated graph (hipGraphExecKernelNodeSetParams)
// before the next replay.  Everything else -- buffers, sizes, layout
// descriptors, the fp16 loss-scale record -- is fixed at capture.
#include <new>
#include <vector>

#include "zr_math.hpp"

struct zr_graph {
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    struct AdamWNode {
        hipGraphNode_t node;
        hipKernelNodeParams params;
        std::vector<void *> args;  // the captured argument pointers; args[index] is replaced
        int index;
    };
    std::vector<AdamWNode> adamw;
    int kernels = 0;
};

namespace zr {
namespace {

std::vector<ScalarSlot> all_slots()
{
    std::vector<ScalarSlot> v(3 * kMaxScalarSlots);
    int k = adamw_scalar_slots(v.data());
    k += fused_scalar_slots(v.data() + k);
    k += fp16_scalar_slots(v.data() + k);
    v.resize(k);
    return v;
}

zr_status hip_fail(const char *who, const char *what, hipError_t e)
{
    return fail(ZR_EHIP, "%s: %s: %s", who, what, hipGetErrorString(e));
}

}  // namespace
}  // namespace zr

using namespace zr;

extern "C" zr_status zr_graph_capture_begin(void *stream)
{
    clear_error();
    if (!stream)
        return fail(ZR_EINVAL, "zr_graph_capture_begin: the null stream cannot be captured");
    hipError_t e = hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal);
    return e == hipSuccess ? ZR_OK : hip_fail("zr_graph_capture_begin", "hipStreamBeginCapture", e);
}

extern "C" zr_status zr_graph_capture_end(void *stream, zr_graph **out)
{
    clear_error();
    const char *who = "zr_graph_capture_end";
    if (!stream || !out)
        return fail(ZR_EINVAL, "%s: NULL stream or out", who);
    *out = nullptr;
    auto *g = new (std::nothrow) zr_graph;
    if (!g) {
        hipGraph_t dropped = nullptr;
        if (hipStreamEndCapture(static_cast<hipStream_t>(stream), &dropped) == hipSuccess && dropped)
            (void)hipGraphDestroy(dropped);
        return fail(ZR_ENOMEM, "%s: out of host memory", who);
    }
    auto bail = [&](zr_status s) {
        zr_graph_destroy(g);
        return s;
    };
    hipError_t e = hipStreamEndCapture(static_cast<hipStream_t>(stream), &g->graph);
    if (e != hipSuccess)
        return bail(hip_fail(who, "hipStreamEndCapture", e));
    if (!g->graph)
        return bail(fail(ZR_EINVAL, "%s: nothing was captured", who));
    size_t count = 0;
    if ((e = hipGraphGetNodes(g->graph, nullptr, &count)) != hipSuccess)
        return bail(hip_fail(who, "hipGraphGetNodes", e));
    std::vector<hipGraphNode_t> nodes(count);
    if (count && (e = hipGraphGetNodes(g->graph, nodes.data(), &count)) != hipSuccess)
        return bail(hip_fail(who, "hipGraphGetNodes", e));
    const std::vector<ScalarSlot> slots = all_slots();
    for (hipGraphNode_t n : nodes) {
        hipGraphNodeType type;
        if ((e = hipGraphNodeGetType(n, &type)) != hipSuccess)
            return bail(hip_fail(who, "hipGraphNodeGetType", e));
        if (type != hipGraphNodeTypeKernel)
            continue;
        ++g->kernels;
        hipKernelNodeParams p{};
        if ((e = hipGraphKernelNodeGetParams(n, &p)) != hipSuccess)
            return bail(hip_fail(who, "hipGraphKernelNodeGetParams", e));
        for (const ScalarSlot &sl : slots) {
            if (sl.func != p.func)
                continue;
            if (!p.kernelParams)
                return bail(fail(ZR_EHIP, "%s: a captured AdamW node has no argument list", who));
            zr_graph::AdamWNode a;
            a.node = n;
            a.params = p;
            a.args.assign(p.kernelParams, p.kernelParams + sl.nargs);
            a.index = sl.index;
            g->adamw.push_back(a);
            break;
        }
    }
    if ((e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0)) != hipSuccess)
        return bail(hip_fail(who, "hipGraphInstantiate", e));
    *out = g;
    return ZR_OK;
}

extern "C" zr_status zr_graph_info(const zr_graph *g, int32_t *kernels, int32_t *adamw_nodes)
{
    clear_error();
    if (!g)
        return fail(ZR_EINVAL, "zr_graph_info: graph is NULL");
    if (kernels)
        *kernels = g->kernels;
    if (adamw_nodes)
        *adamw_nodes = (int32_t)g->adamw.size();
    return ZR_OK;
}

extern "C" zr_status zr_graph_set_adamw(zr_graph *g, const zr_adamw_hparams *hp)
{
    clear_error();
    const char *who = "zr_graph_set_adamw";
    if (!g)
        return fail(ZR_EINVAL, "%s: graph is NULL", who);
    zr_status st = check_adamw_hparams(who, hp);
    if (st != ZR_OK)
        return st;
    AdamWScalars s = adamw_scalars(*hp);
    for (auto &a : g->adamw) {
        std::vector<void *> args = a.args;
        args[a.index] = &s;
        hipKernelNodeParams p = a.params;
        p.kernelParams = args.data();
        p.extra = nullptr;
        hipError_t e = hipGraphExecKernelNodeSetParams(g->exec, a.node, &p);  // copies the arguments
        if (e != hipSuccess)
            return hip_fail(who, "hipGraphExecKernelNodeSetParams", e);
    }
    return ZR_OK;
}

extern "C" zr_status zr_graph_launch(zr_graph *g, void *stream)
{
    clear_error();
    if (!g)
        return fail(ZR_EINVAL, "zr_graph_launch: graph is NULL");
    hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? ZR_OK : hip_fail("zr_graph_launch", "hipGraphLaunch", e);
}

extern "C" void zr_graph_destroy(zr_graph *g)
{
    if (!g)
        return;
    if (g->exec)
        (void)hipGraphExecDestroy(g->exec);
    if (g->graph)
        (void)hipGraphDestroy(g->graph);
    delete g;
}
