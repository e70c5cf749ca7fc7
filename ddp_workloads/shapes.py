"""Parameter shapes of ResNet-50 (He et al., "Deep Residual Learning for Image
Recognition", 2016, Table 1, 50-layer column), in module registration order.

Only the shapes are needed: the gradients are synthetic.  The network is
conv1 (7x7, 3->64) + batch norm, then four stages of 3, 4, 6 and 3 bottleneck
blocks of widths 64, 128, 256 and 512 with expansion 4, then a 2048->1000
fully connected layer.  Each bottleneck registers conv1 (1x1), bn1, conv2
(3x3), bn2, conv3 (1x1), bn3, and its stage's first block also a projection
shortcut: a 1x1 conv and a batch norm.  A batch norm contributes a weight and
a bias (its running statistics are buffers, not parameters).  Convolutions
have no bias.  This gives 161 parameter tensors and 25,557,032 elements.
"""


def resnet50_param_shapes(num_classes=1000):
    """List of (name, shape) in registration order."""
    shapes = [("conv1.weight", (64, 3, 7, 7)),
              ("bn1.weight", (64,)), ("bn1.bias", (64,))]
    inplanes = 64
    for stage, (planes, blocks) in enumerate([(64, 3), (128, 4), (256, 6), (512, 3)], start=1):
        for b in range(blocks):
            pre = f"layer{stage}.{b}."
            shapes += [(pre + "conv1.weight", (planes, inplanes, 1, 1)),
                       (pre + "bn1.weight", (planes,)), (pre + "bn1.bias", (planes,)),
                       (pre + "conv2.weight", (planes, planes, 3, 3)),
                       (pre + "bn2.weight", (planes,)), (pre + "bn2.bias", (planes,)),
                       (pre + "conv3.weight", (planes * 4, planes, 1, 1)),
                       (pre + "bn3.weight", (planes * 4,)), (pre + "bn3.bias", (planes * 4,))]
            if b == 0:
                shapes += [(pre + "downsample.0.weight", (planes * 4, inplanes, 1, 1)),
                           (pre + "downsample.1.weight", (planes * 4,)),
                           (pre + "downsample.1.bias", (planes * 4,))]
            inplanes = planes * 4
    shapes += [("fc.weight", (num_classes, 2048)), ("fc.bias", (num_classes,))]
    return shapes


def resnet50_param_numels(num_classes=1000):
    """Element counts of the parameters, in registration order."""
    out = []
    for _, shape in resnet50_param_shapes(num_classes):
        n = 1
        for d in shape:
            n *= d
        out.append(n)
    return out
