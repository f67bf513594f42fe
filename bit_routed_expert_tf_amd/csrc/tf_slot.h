// Slot-cache internals used by the layer entry point.
#pragma once
#include "tf_internal.h"

tf_status tf_slot_check_layer(const tf_slot_cache *c, const tf_moe_layer *L, int32_t layer);
hipEvent_t tf_slot_fill_event(tf_slot_cache *c);
const int32_t *tf_slot_map(const tf_slot_cache *c, int32_t layer);
const uint8_t *tf_slot_pool(const tf_slot_cache *c, int32_t layer);

// Slot-cache steps planned and filled on the GPU (copy engine
// TF_SLOT_COPY_DEVICE inside tf_moe_layer_fwd): the table view and the
// layer's host and slot blobs.  tf_slot_fused_begin refuses a layer with a
// standalone lookup not yet filled and orders `compute` after the layer's
// last standalone device fill.
struct SlotFused {
    SlotDev d;
    const uint8_t *host_layer;
    uint8_t *slot_layer;
};
bool tf_slot_device_engine(const tf_slot_cache *c);
tf_status tf_slot_fused_begin(tf_slot_cache *c, int32_t layer, hipStream_t compute, SlotFused *out);
